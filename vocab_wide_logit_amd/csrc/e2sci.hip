// E2-SCI adaptive JSD acceptance ("E2-SCI: Elastic Edge-Cloud Speculative
// Decoding via Credit Inertia" notes, key design 3 "online adaptive
// verification"; the credit state of key design 1).
//
// Launch 1: the two-tensor row kernel (asym_rows_kernel with kDeltaNone):
// online softmax statistics of the drafter row y (tensor a) and the target
// row z (tensor b), the team combine, and the JSD terms of each chunk.
// Launch 2, e2sci_finalize_kernel: one wave per row sums the JSD partials
// (D) and tests D <= T of the row's request; the wave that completes a
// request finds the first rejection, updates the credit state
//   r = (1 - beta) r + beta * accept_len / W
// and writes the next window's threshold
//   T = max(T_min, min(T_base + alpha * omega * (r - tau_credit), T_max)).
#include "asym_kernels.hpp"

namespace vwl {

template <int DT>
__global__ __launch_bounds__(kThreads) void e2sci_finalize_kernel(AsymParams P) {
    const int lane = threadIdx.x & 63;
    const long long row = (long long)blockIdx.x * kWaves + (threadIdx.x >> 6);
    if (blockIdx.x == 0 && threadIdx.x == 0)
        P.ctl[0] = 0u; // ticket counter of the row kernel, for the next call
    if (row >= P.R)
        return;
    const uint64_t *rec_row = P.rec + (size_t)row * P.Wmax * kRecWords;
    double jsum = 0.0;
    for (int w = lane; w < P.W; w += 64)
        jsum += as_f64(ld_relaxed(rec_row + (size_t)w * kRecWords + 6));
    jsum = wave_sum(jsum);
    if (lane != 0)
        return;
    const double Dr = -0.5 * kLn2d * jsum;
    const long long bi = row / P.win;
    // the threshold is read before this row's arrival is counted, so the
    // completing wave may overwrite it (thr_out may alias thr_in)
    const uint32_t acc = Dr <= (double)P.thr_in[bi] ? 1u : 0u;
    P.D[row] = (float)Dr;
    P.accept[row] = (uint8_t)acc;
    st_relaxed(P.row_info + (size_t)row * 2 + 1, acc);
    P.row_ctr[(size_t)row * 16] = 0u; // arrivals of the row kernel, for the next call
    uint32_t *rq = P.req_ctr + (size_t)bi * 16;
    const uint32_t done = publish_add(rq, 1u);
    if (done == (uint32_t)(P.win - 1)) {
        const size_t r0 = (size_t)bi * P.win;
        int n = P.win;
        for (int k = 0; k < P.win; ++k) {
            if (ld_relaxed(P.row_info + (r0 + k) * 2 + 1) == 0u) {
                n = k;
                break;
            }
        }
        P.acc_len[bi] = n;
        const double p_acc = (double)n / (double)P.win;
        const double r = (1.0 - P.e_ewma) * (double)P.r_hat[bi] + P.e_ewma * p_acc;
        double T = P.e_Tbase + P.e_alpha * (double)P.omega[bi] * (r - P.e_tau);
        T = T > P.e_Tmax ? P.e_Tmax : T;
        T = T < P.e_Tmin ? P.e_Tmin : T;
        P.r_hat[bi] = (float)r;
        P.thr_out[bi] = (float)T;
        st_relaxed(rq, 0u);
    }
}

template <int DT, int NV>
static hipError_t launch_t(const Plan &plan, const AsymParams &p, hipStream_t s, hipEvent_t after_rows) {
    hipLaunchKernelGGL((asym_rows_kernel<DT, NV, kDeltaNone, kGateCda>), dim3(plan.grid), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (after_rows) {
        e = hipEventRecord(after_rows, s);
        if (e != hipSuccess)
            return e;
    }
    const unsigned fin = (unsigned)((p.R + kWaves - 1) / kWaves);
    hipLaunchKernelGGL((e2sci_finalize_kernel<DT>), dim3(fin), dim3(kThreads), 0, s, p);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_nv(const Plan &plan, const AsymParams &p, hipStream_t s, hipEvent_t after_rows) {
    switch (plan.nv) {
    case 1: return launch_t<DT, 1>(plan, p, s, after_rows);
    case 2: return launch_t<DT, 2>(plan, p, s, after_rows);
    case 4: return launch_t<DT, 4>(plan, p, s, after_rows);
    case 8: return launch_t<DT, 8>(plan, p, s, after_rows);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_e2sci(int dt, const Plan &plan, const AsymParams &p, hipStream_t s, hipEvent_t after_rows) {
    return dt == DT_BF16 ? launch_nv<DT_BF16>(plan, p, s, after_rows) : launch_nv<DT_F32>(plan, p, s, after_rows);
}

template int asym_blocks_per_cu_ds<kDeltaNone>(int dt, int nv, int gate);

} // namespace vwl
