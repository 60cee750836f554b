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
// others' loads and arithmetic; the serial sections (reductions, publish,
// team wait, combine) run at a raised wave priority.
// Launch 2 (the tail): per request, row statistics and the acceptance test
// of each row, the first rejection, then the emitting
// row in fp64 (refined normalisers, the augmented target's log-sum-exp, the
// residual max(p - phat, p - q, 0) or p, and the inverse-CDF draw in
// vocabulary order), phase by phase across the request's workgroups.
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


// Phase-1 exchange of the row kernel without a counter: each member
// publishes its sums of z and y and their references as three words that
// are never zero (a sum's bits with the sign flipped; the two references'
// bits, each with its sign flipped, -0.0 made +0.0 first), so a reader that
// sees a word has its value, with no ordering against other stores.  One
// whole wave polls the team's words and folds them in fixed order: the
// largest reference C, then sum_w s_w 2^(c_w - C) (exact power-of-two
// rescales, since the references are integers; lane w takes members w,
// w + 64, ..., then butterfly sums), so every member gets the same bits;
// the row log-sum-exp is C + log2 of the sum (log2 units).  Returns 2 when
// every word was in at the first look, 1 after waiting, 0 when the wait
// bound expired.
__device__ __forceinline__ uint64_t sum_word(double x) { return f64_bits(x + 0.0) ^ 0x8000000000000000ull; }
__device__ __forceinline__ double word_sum(uint64_t w) { return as_f64(w ^ 0x8000000000000000ull); }
__device__ __forceinline__ uint64_t refs_word(float cz, float cy) {
    return ((uint64_t)(__float_as_uint(cy + 0.0f) ^ 0x80000000u) << 32) |
           (uint64_t)(__float_as_uint(cz + 0.0f) ^ 0x80000000u);
}
__device__ __forceinline__ float word_ref(uint64_t w, bool hi) {
    return __uint_as_float((uint32_t)(hi ? (w >> 32) : w) ^ 0x80000000u);
}
__device__ __forceinline__ uint32_t rapid_poll(const uint64_t *xw, int W, double &Lz2, double &Ly2) {
    const int lane = threadIdx.x & 63;
    uint32_t status = 2u;
    uint64_t t0 = 0;
    float Cz = -3.0e38f, Cy = -3.0e38f;
    uint64_t f0 = 0, f1 = 0, f2 = 0; // the words of member `lane`
    for (int w0 = 0; w0 < W; w0 += 64) {
        const int w = w0 + lane;
        const uint64_t *m = xw + (size_t)w * 4;
        uint64_t v0 = 0, v1 = 0, v2 = 0;
        for (;;) {
            if (w < W) {
                if (v0 == 0)
                    v0 = ld_relaxed(m + 0);
                if (v1 == 0)
                    v1 = ld_relaxed(m + 1);
                if (v2 == 0)
                    v2 = ld_relaxed(m + 2);
            }
            if (__builtin_amdgcn_ballot_w64(w < W && (v0 == 0 || v1 == 0 || v2 == 0)) == 0)
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
            Cz = fmaxf(Cz, word_ref(v2, false));
            Cy = fmaxf(Cy, word_ref(v2, true));
        }
        if (w0 == 0) {
            f0 = v0;
            f1 = v1;
            f2 = v2;
        }
    }
    Cz = wave_max(Cz);
    Cy = wave_max(Cy);
    double sz = 0.0, sy = 0.0;
    for (int w = lane; w < W; w += 64) {
        uint64_t v0 = f0, v1 = f1, v2 = f2;
        if (w >= 64) { // published and final: the reload sees the same words
            const uint64_t *m = xw + (size_t)w * 4;
            v0 = ld_relaxed(m + 0);
            v1 = ld_relaxed(m + 1);
            v2 = ld_relaxed(m + 2);
        }
        sz += scale_pow2(word_sum(v0), word_ref(v2, false) - Cz);
        sy += scale_pow2(word_sum(v1), word_ref(v2, true) - Cy);
    }
    sz = wave_sum(sz);
    sy = wave_sum(sy);
    Lz2 = (double)Cz + log2(sz);
    Ly2 = (double)Cy + log2(sy);
    return status;
}

// Online sum-of-exp state of one tensor over a thread's elements, fed one
// 16-byte group of raw logits x at a time, for the exponent x*c (log2 units,
// c = log2e/T).  The product is evaluated as an fma with the reference
// subtracted before rounding, plus the low part of c, so no rounding of x/T
// or of x*c at the logits' magnitude enters the exponent.  The reference is
// an integer at or above the running maximum, so the state means
// s = sum_v 2^(x_v*c - ref) exactly as evaluated, and a change of reference
// is an exact power-of-two rescale.
struct OnlineLseR {
    float c;   // reference, log2 units, integer-valued
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
    // finite even for -inf rows (the high part of c is positive)
    const float c_new = fmaxf(st.c, __builtin_ceilf(fmaxf(g, -1e30f) * k.hi));
    float acc = __builtin_amdgcn_exp2f(scaled_arg(x[0], k, c_new));
#pragma unroll
    for (int e = 1; e < EPV; ++e)
        acc += __builtin_amdgcn_exp2f(scaled_arg(x[e], k, c_new));
    st.s = scale_pow2(st.s, st.c - c_new) + (double)acc;
    st.c = c_new;
}

// Rescale a thread's state to the workgroup reference C (fp64, exact).
__device__ __forceinline__ double rescale_to_r(const OnlineLseR &st, float C) {
    return scale_pow2(st.s, st.c - C);
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
    const float c_new = fmaxf(st.c, __builtin_ceilf(fmaxf(g, -1e30f)));
    float acc = __builtin_amdgcn_exp2f(aug_harg(k, z[0], dqp[0], c_new));
#pragma unroll
    for (int e = 1; e < EPV; ++e)
        acc += __builtin_amdgcn_exp2f(aug_harg(k, z[e], dqp[e], c_new));
    st.s = scale_pow2(st.s, st.c - c_new) + (double)acc;
    st.c = c_new;
}

__device__ __forceinline__ void split_f64(double x, float &hi, float &lo) {
    hi = (float)x;
    lo = (float)(x - (double)hi);
}

// Reductions within the 16-lane segment of a wave that holds one row.
__device__ __forceinline__ float seg16_max(float v) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1)
        v = fmaxf(v, __shfl_xor(v, m, 16));
    return v;
}
__device__ __forceinline__ double seg16_sum(double v) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1)
        v += __shfl_xor(v, m, 16);
    return v;
}
__device__ __forceinline__ int seg16_min_int(int v) {
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1)
        v = min(v, __shfl_xor(v, m, 16));
    return v;
}

// Row statistics and the acceptance test of one row, by one 16-lane segment
// of a wave (so a wave handles four rows at once): all record words of the
// row are loaded in one round.  The segment's lane 0 leaves L_z, L_y, Mhat,
// L_zhat, the argmax and the acceptance flag in `slot`; with `write` it
// also stores the row's outputs and clears the row kernel's published words
// of the row.  Every
// lane of the segment must call it (the reductions are segment-wide).
template <int DT>
__device__ __forceinline__ void tail_row(const RapidParams &P, long long row, bool write, double *slot) {
    const int lane = threadIdx.x & 15;
    const int Pn = P.G + 1;
    const long long bi = row / Pn;
    const int i = (int)(row - bi * Pn);
    const size_t row_off = (size_t)row * (size_t)P.V;
    // the draft's logits, early (independent of the records)
    int x = -1;
    double zx = 0.0, yx = 0.0;
    if (i < P.G) {
        x = P.draft[bi * P.G + i];
        if (lane == 0 && x >= 0 && x < P.V) {
            zx = (double)load_scalar<DT>(P.z, row_off + x) * P.invT64;
            yx = (double)load_scalar<DT>(P.y, row_off + x) * P.invT64;
        }
    }
    const uint64_t *rec_row = P.rec + (size_t)row * P.Wmax * kRecWords;
    const float NEG = -3.0e38f;
    float cz = NEG, cy = NEG, ch = NEG, mh = -__builtin_inff();
    double sz = 0.0, sy = 0.0, sh = 0.0;
    int hidx = 0x7fffffff;
    // first pass: references and the maximum (loads kept for the second)
    uint64_t w0[2] = {0, 0}, w1[2] = {0, 0}, w2[2] = {0, 0}, w3[2] = {0, 0}, w4[2] = {0, 0}, w5[2] = {0, 0};
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const int w = lane + 16 * k;
        if (w < P.W) {
            const uint64_t *r = rec_row + (size_t)w * kRecWords;
            w0[k] = ld_relaxed(r + 0);
            w1[k] = ld_relaxed(r + 1);
            w2[k] = ld_relaxed(r + 2);
            w3[k] = ld_relaxed(r + 3);
            w4[k] = ld_relaxed(r + 4);
            w5[k] = ld_relaxed(r + 5);
        }
    }
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (lane + 16 * k < P.W) {
            cz = fmaxf(cz, unpack_lo(w2[k]));
            cy = fmaxf(cy, unpack_hi(w2[k]));
            ch = fmaxf(ch, unpack_lo(w5[k]));
            const float m = unpack_lo(w4[k]);
            const int ix = (int)(uint32_t)(w4[k] >> 32);
            if (m > mh || (m == mh && ix < hidx)) {
                mh = m;
                hidx = ix;
            }
        }
    }
    for (int w = lane + 32; w < P.W; w += 16) { // teams wider than 32 members
        const uint64_t *r = rec_row + (size_t)w * kRecWords;
        const uint64_t a2 = ld_relaxed(r + 2), a4 = ld_relaxed(r + 4), a5 = ld_relaxed(r + 5);
        cz = fmaxf(cz, unpack_lo(a2));
        cy = fmaxf(cy, unpack_hi(a2));
        ch = fmaxf(ch, unpack_lo(a5));
        const float m = unpack_lo(a4);
        const int ix = (int)(uint32_t)(a4 >> 32);
        if (m > mh || (m == mh && ix < hidx)) {
            mh = m;
            hidx = ix;
        }
    }
    cz = seg16_max(cz);
    cy = seg16_max(cy);
    ch = seg16_max(ch);
    const float mh_all = seg16_max(mh);
    hidx = seg16_min_int(mh == mh_all ? hidx : 0x7fffffff);
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        if (lane + 16 * k < P.W) {
            sz += scale_pow2(as_f64(w0[k]), unpack_lo(w2[k]) - cz);
            sy += scale_pow2(as_f64(w1[k]), unpack_hi(w2[k]) - cy);
            sh += scale_pow2(as_f64(w3[k]), unpack_lo(w5[k]) - ch);
        }
    }
    for (int w = lane + 32; w < P.W; w += 16) {
        const uint64_t *r = rec_row + (size_t)w * kRecWords;
        const uint64_t a2 = ld_relaxed(r + 2), a5 = ld_relaxed(r + 5);
        sz += scale_pow2(as_f64(ld_relaxed(r + 0)), unpack_lo(a2) - cz);
        sy += scale_pow2(as_f64(ld_relaxed(r + 1)), unpack_hi(a2) - cy);
        sh += scale_pow2(as_f64(ld_relaxed(r + 3)), unpack_lo(a5) - ch);
    }
    sz = seg16_sum(sz);
    sy = seg16_sum(sy);
    sh = seg16_sum(sh);
    if (write) { // the row kernel's published words back to zero, for the next call
        for (int w = lane; w < P.W; w += 16) {
            uint64_t *xw = P.xw + ((size_t)row * P.Wmax + w) * 4;
            st_relaxed(xw + 0, 0ull);
            st_relaxed(xw + 1, 0ull);
            st_relaxed(xw + 2, 0ull);
        }
    }
    if (lane != 0)
        return;
    const double Lz = ((double)cz + log2(sz)) * kLn2d;
    const double Ly = ((double)cy + log2(sy)) * kLn2d;
    const double Lh = ((double)ch + log2(sh)) * kLn2d;
    const double eta_d = P.eta_d;
    // Mhat: the augmented logit at the argmax, recomputed in fp64
    double Mh = (double)mh_all * kLn2d;
    if (hidx >= 0 && hidx < P.V) {
        const double zm = (double)load_scalar<DT>(P.z, row_off + hidx) * P.invT64;
        const double ym = (double)load_scalar<DT>(P.y, row_off + hidx) * P.invT64;
        Mh = zm + eta_d * (exp(ym - Ly) - exp(zm - Lz));
    } else {
        hidx = -1;
    }
    slot[0] = Lz;
    slot[1] = Ly;
    slot[2] = Mh;
    slot[3] = Lh;
    slot[4] = (double)hidx;
    if (write) {
        double *rs = P.rowstat + (size_t)row * kRowStatWords;
        st_f64(rs + 0, Lz);
        st_f64(rs + 1, Ly);
        st_f64(rs + 2, Mh);
        st_f64(rs + 3, Lh);
        st_f64(rs + 4, (double)hidx);
    }
    uint32_t acc = 0;
    if (i < P.G) {
        const long long k = bi * P.G + i;
        float phd = 0.f, qd = 0.f;
        if (x < 0 || x >= P.V) {
            if (write)
                set_dev_err(P.dev_err, 1);
        } else {
            const double p = exp(zx - Lz);
            const double q = exp(yx - Ly);
            const double h = zx + eta_d * (q - p);
            const double ph = (h - Mh < -2.302585092994046) ? p : exp(h - Lh);
            const double u = clamp_uniform(P.u_accept[k], write ? P.dev_err : nullptr);
            acc = (u * q < ph) ? 1u : 0u;
            phd = (float)ph;
            qd = (float)q;
        }
        if (write) {
            P.accept[k] = (uint8_t)acc;
            if (P.p_hat_draft)
                P.p_hat_draft[k] = phd;
            if (P.q_draft)
                P.q_draft[k] = qd;
        }
    }
    slot[5] = (double)acc;
}

template <int DT, int NV>
__global__ __launch_bounds__(kThreads, (NV <= 4 ? 5 : 4)) void rapid_rows_kernel(RapidParams P) {
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
        OnlineLseR lz{-3.0e38f, 0.0}, ly{-3.0e38f, 0.0};
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
        __builtin_amdgcn_s_setprio(2); // serial section: reductions, publish, team wait, combine
        block_max<2>(mx, lds_f);
        double S[2] = {rescale_to_r(lz, mx[0]), rescale_to_r(ly, mx[1])};
        block_sum<2>(S, lds_d);

        if (tid == 0) {
            uint64_t *rec = P.rec + ((size_t)row * P.Wmax + member) * kRecWords;
            st_relaxed(rec + 0, f64_bits(S[0]));
            st_relaxed(rec + 1, f64_bits(S[1]));
            st_relaxed(rec + 2, (uint64_t)__float_as_uint(mx[0]) | ((uint64_t)__float_as_uint(mx[1]) << 32));
            uint64_t *xw = P.xw + ((size_t)row * P.Wmax + member) * 4;
            st_relaxed(xw + 0, sum_word(S[0]));
            st_relaxed(xw + 1, sum_word(S[1]));
            st_relaxed(xw + 2, refs_word(mx[0], mx[1]));
        }
        if (tid < 64) {
            double Lz2 = 0.0, Ly2 = 0.0;
            const uint32_t st = rapid_poll(P.xw + (size_t)row * P.Wmax * 4, P.W, Lz2, Ly2);
            if (tid == 0) {
                sh_row[0] = Lz2;
                sh_row[1] = Ly2;
                sh_u[1] = st;
            }
        }
        __syncthreads();
        if (!sh_u[1]) {
            if (tid == 0)
                set_dev_err(P.dev_err, 4);
            return;
        }
        __builtin_amdgcn_s_setprio(0);

        // ---- second pass: h = zhat/T = z/T + eta*(q - p); online statistics ----
        AugCoef ak;
        ak.c = kc;
        split_f64(sh_row[0], ak.lz_hi, ak.lz_lo);
        split_f64(sh_row[1], ak.ly_hi, ak.ly_lo);
        ak.eta2 = P.eta2;
        OnlineLseR lh{-3.0e38f, 0.0};
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
        __builtin_amdgcn_s_setprio(2);
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
            st_relaxed(rec + 3, f64_bits(Sh[0]));
            st_relaxed(rec + 4, pack_fi(Hm, hi));
            st_relaxed(rec + 5, (uint64_t)__float_as_uint(Ch));
        }
        __builtin_amdgcn_s_setprio(0);
    }
}

// ---------------------------------------------------------------------------
// Launch 2, the tail: one team of We workgroups per request; workgroup w
// owns the EPT * 256 elements of the request's emitting row starting at
// w * EPT * 256 (EPT contiguous elements per thread).  Every workgroup
// combines the records of all the request's rows (row statistics, Mhat in
// fp64 at the argmax, the draft's tail-protected phat and q and the
// acceptance test, one row per 16-lane segment; workgroup 0 writes them
// out), so each knows the accept
// length n and the emitting row's statistics at once.  Phases, separated by
// barriers of the request's team:
//   1  per element, around the row pass's log-sum-exps,
//      p' = exp(z/T - L_z), q' = exp(y/T - L_y), h' = z/T + eta (q' - p')
//      and e' = exp(h' - M) (M the row pass's maximum of h), kept in
//      registers -> chunk sums of p', q', e', e'q', e'p'.
//   2  (residual rows) the refined normalisers f_z = 1 / sum p', f_y =
//      1 / sum q' make p = f_z p' and q = f_y q' sum to one; they move h by
//      d = eta (q' (f_y - 1) - p' (f_z - 1)), of the order of the row
//      pass's rounding (1e-7 relative), so sum exp(h - M) = sum e' + eta
//      (f_y - 1) sum e'q' - eta (f_z - 1) sum e'p' to second order in d and
//      phat = e' exp(d) / that sum; Mhat is recomputed in fp64 at the
//      argmax.  Residual max(p - phat, p - q, 0) per element -> chunk sums.
//   3  the chunk that holds u * S walks its elements in vocabulary order;
//      emit_dist when requested.
// A bonus row (n = G) draws from p, whose normalisation does not move the
// draw, so it goes from phase 1 (sums of p') straight to phase 3.
// Chunk intervals come from one fixed-order running sum evaluated the same
// way by every workgroup, so they tile [0, S) exactly.  Everything on the
// emitting row is fp64, with three exponentials per element.
// With n < G the residual of row n is drawn from (p of row n when the
// residual is all zero); with n = G, p of the bonus row.
// Per-request partials [B][We][8]: 0 residual weights, 1 p, 2 e', 3 p',
// 4 q', 5 e'q', 6 e'p'.
// ---------------------------------------------------------------------------

// Barrier of a request's team: every wave's stores complete, one arrival
// per workgroup, wait for `target` arrivals.  Returns false on timeout.
__device__ __forceinline__ bool tail_sync(uint32_t *ctr, uint32_t target, uint32_t *sh_flag) {
    wait_stores_complete();
    __syncthreads();
    if (threadIdx.x == 0) {
        publish_add_nr(ctr, 1u);
        *sh_flag = wait_at_least(ctr, target) ? 1u : 0u;
    }
    __syncthreads();
    return *sh_flag != 0u;
}

// Sums of NW words of the request's We partials, each in one fixed order, the
// same in every workgroup: lane l of wave 0 adds up the partials
// [l*m, (l+1)*m) in index order (m = ceil(We/64)); the lane totals are then
// added in lane order.  When w >= 0 also returns E(w) and E(w + 1) of each
// word, where E(k) is the same fixed-order sum over the partials before chunk
// k, so the intervals [E(k), E(k+1)) of all chunks tile [0, E(We)) exactly.
template <int NW>
__device__ __forceinline__ void tail_parts(const double *parts, int We, const int (&word)[NW],
                                           double *sh_lane /* 3*64*NW */, double *sh_out /* 3*NW */, int w,
                                           double (&total)[NW], double (&pre0)[NW], double (&pre1)[NW]) {
    const int tid = threadIdx.x;
    if (tid < 64) {
        const int m = (We + 63) / 64;
        const int k0 = tid * m, k1 = min(k0 + m, We);
        double c[NW], e0[NW], e1[NW];
#pragma unroll
        for (int j = 0; j < NW; ++j)
            c[j] = e0[j] = e1[j] = 0.0;
        for (int k = k0; k < k1; ++k) {
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                if (k == w)
                    e0[j] = c[j];
                c[j] += ld_f64(parts + (size_t)k * kEmitWords + word[j]);
                if (k == w)
                    e1[j] = c[j];
            }
        }
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            sh_lane[(3 * j) * 64 + tid] = c[j];
            sh_lane[(3 * j + 1) * 64 + tid] = e0[j];
            sh_lane[(3 * j + 2) * 64 + tid] = e1[j];
        }
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (tid == 0) {
            double t[NW], a0[NW], a1[NW];
#pragma unroll
            for (int j = 0; j < NW; ++j)
                t[j] = a0[j] = a1[j] = 0.0;
            const int lw = (w >= 0) ? w / m : -1;
            for (int l = 0; l < 64; ++l) {
#pragma unroll
                for (int j = 0; j < NW; ++j) {
                    if (l == lw) {
                        a0[j] = t[j] + sh_lane[(3 * j + 1) * 64 + l];
                        a1[j] = t[j] + sh_lane[(3 * j + 2) * 64 + l];
                    }
                    t[j] += sh_lane[(3 * j) * 64 + l];
                }
            }
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                sh_out[3 * j] = t[j];
                sh_out[3 * j + 1] = a0[j];
                sh_out[3 * j + 2] = a1[j];
            }
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        total[j] = sh_out[3 * j];
        pre0[j] = sh_out[3 * j + 1];
        pre1[j] = sh_out[3 * j + 2];
    }
    __syncthreads();
}

// Partial sums exchanged between a request's workgroups as self-validating
// words: a published sum x >= 0 is stored as the bits of x + 0.0 with the
// sign bit flipped, which is never zero, and a word still zero has not been
// published yet; so a reader polls the words themselves (one round trip, no
// arrival counter).  The request's last workgroup to leave clears them.
__device__ __forceinline__ uint64_t part_word(double x) {
    return static_cast<uint64_t>(__double_as_longlong(x + 0.0)) ^ 0x8000000000000000ull;
}
__device__ __forceinline__ double part_value(uint64_t u) { return as_f64(u ^ 0x8000000000000000ull); }

// As tail_parts, with each lane of wave 0 waiting for the words it sums to
// be published; returns false (in every thread) when a wait exceeds the
// bound.  Called by the whole workgroup.
template <int NW>
__device__ __forceinline__ bool tail_parts_poll(const double *parts, int We, const int (&word)[NW],
                                                double *sh_lane /* 3*64*NW */, double *sh_out /* 3*NW */,
                                                uint32_t *sh_flag, int w, double (&total)[NW], double (&pre0)[NW],
                                                double (&pre1)[NW]) {
    const int tid = threadIdx.x;
    if (tid < 64) {
        const int m = (We + 63) / 64;
        const int k0 = tid * m, k1 = min(k0 + m, We);
        double c[NW], e0[NW], e1[NW];
#pragma unroll
        for (int j = 0; j < NW; ++j)
            c[j] = e0[j] = e1[j] = 0.0;
        bool ok = true;
        uint64_t t0 = 0;
        for (int k = k0; k < k1 && ok; ++k) {
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                const uint64_t *a = reinterpret_cast<const uint64_t *>(parts + (size_t)k * kEmitWords + word[j]);
                uint64_t u = ld_relaxed(a);
                while (u == 0u && ok) {
                    if (t0 == 0)
                        t0 = wall_clock64();
                    __builtin_amdgcn_s_sleep(1);
                    u = ld_relaxed(a);
                    if (u == 0u && wall_clock64() - t0 > kWaitLimitTicks)
                        ok = false;
                }
                if (k == w)
                    e0[j] = c[j];
                c[j] += part_value(u);
                if (k == w)
                    e1[j] = c[j];
            }
        }
#pragma unroll
        for (int j = 0; j < NW; ++j) {
            sh_lane[(3 * j) * 64 + tid] = c[j];
            sh_lane[(3 * j + 1) * 64 + tid] = e0[j];
            sh_lane[(3 * j + 2) * 64 + tid] = e1[j];
        }
        const bool all_ok = __all(ok);
        __asm__ volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        if (tid == 0) {
            double t[NW], a0[NW], a1[NW];
#pragma unroll
            for (int j = 0; j < NW; ++j)
                t[j] = a0[j] = a1[j] = 0.0;
            const int lw = (w >= 0) ? w / m : -1;
            for (int l = 0; l < 64; ++l) {
#pragma unroll
                for (int j = 0; j < NW; ++j) {
                    if (l == lw) {
                        a0[j] = t[j] + sh_lane[(3 * j + 1) * 64 + l];
                        a1[j] = t[j] + sh_lane[(3 * j + 2) * 64 + l];
                    }
                    t[j] += sh_lane[(3 * j) * 64 + l];
                }
            }
#pragma unroll
            for (int j = 0; j < NW; ++j) {
                sh_out[3 * j] = t[j];
                sh_out[3 * j + 1] = a0[j];
                sh_out[3 * j + 2] = a1[j];
            }
            *sh_flag = all_ok ? 1u : 0u;
        }
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < NW; ++j) {
        total[j] = sh_out[3 * j];
        pre0[j] = sh_out[3 * j + 1];
        pre1[j] = sh_out[3 * j + 2];
    }
    const bool ok = *sh_flag != 0u;
    __syncthreads();
    return ok;
}

template <int DT, int EPT>
__global__ __launch_bounds__(kThreads, (EPT <= 8 ? 4 : 3)) void rapid_tail_kernel(RapidParams P) {
    __shared__ double lds_d[kWaves * 5];
    __shared__ int lds_i[kWaves];
    __shared__ double sh_lane[3 * 64 * 5];
    __shared__ double sh_out[3 * 5];
    __shared__ double sh_st[4];
    __shared__ double sh_scan[kWaves];
    __shared__ double sh_rows[(kMaxDrafts + 1) * 6];
    __shared__ uint32_t sh_u[2];
    const int tid = threadIdx.x;
    const int We = P.We;
    const int bi = (int)(blockIdx.x / (unsigned)We), w = (int)(blockIdx.x % (unsigned)We);
    const int Pn = P.G + 1;
    if (blockIdx.x == 0 && tid == 0)
        P.ctl[0] = 0u; // ticket counter of the row kernel, for the next call
    uint32_t *leave = P.req_ctr + (size_t)bi * 16 + 5;
    double *parts = P.emit + (size_t)bi * We * kEmitWords;
    uint64_t *mine = reinterpret_cast<uint64_t *>(parts + (size_t)w * kEmitWords);
    bool ok = true;

    // ---- the request's rows: statistics and acceptance, in every
    // workgroup (one wave per row; workgroup 0 also writes the outputs), so
    // each finds the accept length and the emitting row without a barrier ----
    for (int r0 = (tid >> 6) * 4; r0 < Pn; r0 += kWaves * 4) {
        const int r = r0 + ((tid & 63) >> 4);
        if (r < Pn) // whole 16-lane segments
            tail_row<DT>(P, (long long)bi * Pn + r, w == 0, sh_rows + r * 6);
    }
    __syncthreads();
    if (tid == 0) {
        int first = P.G;
        for (int k = 0; k < P.G; ++k)
            if (sh_rows[k * 6 + 5] == 0.0) {
                first = k;
                break;
            }
        sh_u[1] = (uint32_t)first;
    }
    __syncthreads();
    const int n = (int)sh_u[1];
    if (w == 0 && tid == 0)
        P.acc_len[bi] = n;
    const long long row = (long long)bi * Pn + n;
    const size_t row_off = (size_t)row * (size_t)P.V;
    const bool resid = n < P.G;
    const double *rs = sh_rows + n * 6;
    const int v0 = (w * kThreads + tid) * EPT;
    const double invT = P.invT64, eta_d = P.eta_d;
    const double Lz = rs[0], Ly = rs[1], Mr = rs[2];

    // z and y at the augmented argmax (for Mhat), fetched early by thread 0
    int hidx = -1;
    double zxh = 0.0, yxh = 0.0;
    if (tid == 0) {
        hidx = (int)rs[4];
        if (resid && hidx >= 0 && hidx < P.V) {
            zxh = (double)load_scalar<DT>(P.z, row_off + hidx) * invT;
            yxh = (double)load_scalar<DT>(P.y, row_off + hidx) * invT;
        }
    }

    // ---- phase 1: p', q', e' per element, kept; chunk sums ----
    double pc[EPT], qc[EPT], ec[EPT];
    float zc[EPT];
#pragma unroll
    for (int e = 0; e < EPT; ++e) {
        pc[e] = qc[e] = ec[e] = 0.0;
        zc[e] = 0.0f;
    }
    if (resid) {
        double s5[5] = {0.0, 0.0, 0.0, 0.0, 0.0};
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int v = v0 + e;
            if (v < P.V) {
                zc[e] = load_scalar<DT>(P.z, row_off + v);
                const double zs = (double)zc[e] * invT;
                pc[e] = exp(zs - Lz);
                qc[e] = exp((double)load_scalar<DT>(P.y, row_off + v) * invT - Ly);
                ec[e] = exp(zs + eta_d * (qc[e] - pc[e]) - Mr);
                s5[0] += pc[e];
                s5[1] += qc[e];
                s5[2] += ec[e];
                s5[3] += ec[e] * qc[e];
                s5[4] += ec[e] * pc[e];
            }
        }
        block_sum<5>(s5, lds_d);
        if (tid == 0) {
            st_relaxed(mine + 3, part_word(s5[0]));
            st_relaxed(mine + 4, part_word(s5[1]));
            st_relaxed(mine + 2, part_word(s5[2]));
            st_relaxed(mine + 5, part_word(s5[3]));
            st_relaxed(mine + 6, part_word(s5[4]));
        }
    } else {
        double s1[1] = {0.0};
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            const int v = v0 + e;
            if (v < P.V) {
                pc[e] = exp((double)load_scalar<DT>(P.z, row_off + v) * invT - Lz);
                s1[0] += pc[e];
            }
        }
        block_sum<1>(s1, lds_d);
        if (tid == 0)
            st_relaxed(mine + 3, part_word(s1[0]));
    }

    // ---- phase 2 (residual rows): refined factors, residual sums ----
    double fz = 1.0, fy = 1.0, Mh = 0.0, iE = 0.0;
    if (resid) {
        double t5[5], unused0[5], unused1[5];
        ok = tail_parts_poll<5>(parts, We, {3, 4, 2, 5, 6}, sh_lane, sh_out, &sh_u[0], -1, t5, unused0, unused1);
        if (tid == 0) {
            const double gz = 1.0 / t5[0], gy = 1.0 / t5[1];
            double mh = Mr;
            if (hidx >= 0 && hidx < P.V)
                mh = zxh + eta_d * (exp(yxh - Ly) * gy - exp(zxh - Lz) * gz);
            // sum of exp(h - M) over the row with h = h' + d, to first order in d
            const double E = t5[2] + eta_d * ((gy - 1.0) * t5[3] - (gz - 1.0) * t5[4]);
            sh_st[0] = gz;
            sh_st[1] = gy;
            sh_st[2] = mh;
            sh_st[3] = 1.0 / E;
        }
        __syncthreads();
        fz = sh_st[0];
        fy = sh_st[1];
        Mh = sh_st[2];
        iE = sh_st[3];
    }

    // weights of element e: residual max(p - phat, p - q, 0), or p' for a
    // bonus row (the draw normalises by the sum)
    auto weights = [&](int e, double &r, double &p) {
        if (!resid) {
            p = pc[e];
            r = 0.0;
            return;
        }
        p = pc[e] * fz;
        const double q = qc[e] * fy;
        const double d = eta_d * (qc[e] * (fy - 1.0) - pc[e] * (fz - 1.0));
        const double h = (double)zc[e] * invT + eta_d * (qc[e] - pc[e]) + d;
        const double ph = (h - Mh < -2.302585092994046) ? p : ec[e] * (1.0 + d * (1.0 + 0.5 * d)) * iE;
        double dd = p - ph;
        if (p - q > dd)
            dd = p - q;
        r = dd > 0.0 ? dd : 0.0;
    };

    if (ok && resid) {
        double s2[2] = {0.0, 0.0};
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            if (v0 + e < P.V) {
                double r, p;
                weights(e, r, p);
                s2[0] += r;
                s2[1] += p;
            }
        }
        block_sum<2>(s2, lds_d);
        if (tid == 0) {
            st_relaxed(mine + 0, part_word(s2[0]));
            st_relaxed(mine + 1, part_word(s2[1]));
        }
    }

    // ---- phase 3: the draw ----
    // residual (word 0) and target (word 1) sums with this chunk's interval;
    // a bonus row's target sums are word 3
    double St[2] = {0.0, 0.0}, e0[2] = {0.0, 0.0}, e1[2] = {0.0, 0.0};
    if (ok) {
        if (resid) {
            ok = tail_parts_poll<2>(parts, We, {0, 1}, sh_lane, sh_out, &sh_u[0], w, St, e0, e1);
        } else {
            double t1[1], a0[1], a1[1];
            ok = tail_parts_poll<1>(parts, We, {3}, sh_lane, sh_out, &sh_u[0], w, t1, a0, a1);
            St[0] = 0.0;
            St[1] = t1[0];
            e0[0] = e1[0] = 0.0;
            e0[1] = a0[0];
            e1[1] = a1[0];
        }
    }
    if (ok) {
        const bool use_r = resid && (St[0] > 0.0);
        const double S = use_r ? St[0] : St[1];
        const double pre0 = use_r ? e0[0] : e0[1], pre1 = use_r ? e1[0] : e1[1];
        const double u = clamp_uniform(P.u_sample[row], (w == 0 && tid == 0) ? P.dev_err : nullptr);
        const double target = u * S;
        const bool crossing_here = (pre0 <= target) && (target < pre1);
        double wt[EPT];
        double tsum = 0.0;
#pragma unroll
        for (int e = 0; e < EPT; ++e) {
            double r = 0.0, p = 0.0;
            if (v0 + e < P.V)
                weights(e, r, p);
            wt[e] = use_r ? r : p;
            tsum += wt[e];
        }
        if (P.emit_dist) {
            const double invS = 1.0 / S;
#pragma unroll
            for (int e = 0; e < EPT; ++e)
                if (v0 + e < P.V)
                    P.emit_dist[(size_t)bi * P.V + v0 + e] = (float)(wt[e] * invS);
        }
        if (crossing_here) {
            // exclusive scan of the per-thread sums in thread order: within
            // each wave by lane shifts (fixed order), then the wave totals
            const int lane = tid & 63, wave = tid >> 6;
            double x = tsum;
#pragma unroll
            for (int o = 1; o < 64; o <<= 1) {
                const double y = __shfl_up(x, o, 64);
                if (lane >= o)
                    x += y;
            }
            double excl = __shfl_up(x, 1, 64);
            if (lane == 0)
                excl = 0.0;
            if (lane == 63)
                sh_scan[wave] = x;
            __syncthreads();
            double off = pre0;
            for (int k = 0; k < wave; ++k)
                off += sh_scan[k];
            int found = 0x7fffffff, last_pos = -1;
            double c = off + excl;
#pragma unroll
            for (int e = 0; e < EPT; ++e) {
                const int v = v0 + e;
                if (v < P.V) {
                    c += wt[e];
                    if (wt[e] > 0.0)
                        last_pos = v;
                    if (c > target && found == 0x7fffffff)
                        found = v;
                }
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
    }
    if (!ok && tid == 0)
        set_dev_err(P.dev_err, 4);

    // the request's last workgroup to leave (every other one has read all
    // the partials it needs) clears the partial words and the counter
    __syncthreads();
    if (tid == 0)
        sh_u[1] = publish_add(leave, 1u) == (uint32_t)We - 1u ? 1u : 0u;
    __syncthreads();
    if (sh_u[1] != 0u) {
        uint64_t *all = reinterpret_cast<uint64_t *>(parts);
        for (int k = tid; k < We * kEmitWords; k += kThreads)
            st_relaxed(all + k, 0ull);
        if (tid == 0)
            st_relaxed(leave, 0u);
    }
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
    const dim3 tg((unsigned)p.We * (unsigned)p.B);
    if (p.ept <= 8)
        hipLaunchKernelGGL((rapid_tail_kernel<DT, 8>), tg, dim3(kThreads), 0, s, p);
    else
        hipLaunchKernelGGL((rapid_tail_kernel<DT, 16>), tg, dim3(kThreads), 0, s, p);
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
