// Passes built on the two-tensor divergence kernel (asym_rows_kernel with
// kDeltaNone): E2-SCI's adaptive acceptance and AsymSpec across model
// families.
//
// E2-SCI adaptive JSD acceptance ("E2-SCI: Elastic Edge-Cloud Speculative
// Decoding via Credit Inertia" notes, key design 3 "online adaptive
// verification"; the credit state of key design 1).
//
// Launch 1: the two-tensor row kernel (asym_rows_kernel with kDeltaNone):
// online softmax statistics of the drafter row y (tensor a) and the target
// row z (tensor b), the team combine, and the JSD terms of each chunk.
// Launch 2, e2sci_finalize_kernel: one workgroup per request; one wave per
// row sums the JSD partials (D) and tests D <= T of the request; then one
// thread finds the first rejection, updates the credit state
//   r = (1 - beta) r + beta * accept_len / W
// and writes the next window's threshold
//   T = max(T_min, min(T_base + alpha * omega * (r - tau_credit), T_max)),
// passed through the stabilisers of the same passage: an accepted fraction
// below delta falls back to T_safe; otherwise the current threshold is kept
// while it has been in effect for fewer than min_refresh windows or while
// the proposal lies within the hysteresis band of it.
#include "asym_kernels.hpp"

namespace vwl {

template <int DT>
__global__ __launch_bounds__(kFinMaxThreads) void e2sci_finalize_kernel(AsymParams P) {
    __shared__ uint32_t sh_acc[kMaxDrafts + 1]; // a window holds at most VWL_MAX_K + 1 rows
    const int lane = threadIdx.x & 63;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        P.ctl[0] = 0u; // ticket counter of the row kernel, for the next call
    const long long bi = blockIdx.x;
    const double T_cur = (double)P.thr_in[bi];
    // the request's credit state, in flight while the rows are combined
    float r_in = 0.0f, om = 0.0f;
    int age_in = 0;
    if (threadIdx.x == 0) {
        r_in = P.r_hat[bi];
        om = P.omega[bi];
        age_in = P.age ? P.age[bi] : 0;
    }
    for (int i = (int)(threadIdx.x >> 6); i < P.win; i += (int)(blockDim.x >> 6)) {
        const long long row = bi * P.win + i;
        const uint64_t *rec_row = P.rec + (size_t)row * P.Wmax * kRecWords;
        double jsum = 0.0;
        for (int w = lane; w < P.W; w += 64)
            jsum += as_f64(ld_relaxed(rec_row + (size_t)w * kRecWords + 6));
        jsum = wave_sum(jsum);
        clear_row_exchange(P, row);
        if (lane == 0) {
            const uint32_t acc = jsum <= T_cur ? 1u : 0u;
            P.D[row] = (float)jsum;
            P.accept[row] = (uint8_t)acc;
            sh_acc[i] = acc;
        }
    }
    __syncthreads();
    if (threadIdx.x != 0)
        return;
    int n = P.win;
    for (int k = 0; k < P.win; ++k) {
        if (sh_acc[k] == 0u) {
            n = k;
            break;
        }
    }
    P.acc_len[bi] = n;
    const double p_acc = (double)n / (double)P.win;
    const double r = (1.0 - P.e_ewma) * (double)r_in + P.e_ewma * p_acc;
    double T = P.e_Tbase + P.e_alpha * (double)om * (r - P.e_tau);
    T = T > P.e_Tmax ? P.e_Tmax : T;
    T = T < P.e_Tmin ? P.e_Tmin : T;
    // stabilisers: safety fall-back, minimum refresh interval, dead band
    const int age_next = age_in < 0x7fffffff ? age_in + 1 : age_in;
    int age_out = 0;
    if (p_acc < P.e_delta) {
        T = P.e_Tsafe;
    } else if (age_next < P.e_minref || !(fabs(T - T_cur) > P.e_hyst)) {
        T = T_cur;
        age_out = age_next;
    }
    if (P.age)
        P.age[bi] = age_out;
    P.r_hat[bi] = (float)r;
    P.thr_out[bi] = (float)T; // thr_out may alias thr_in: every row has been tested above
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
    hipLaunchKernelGGL((e2sci_finalize_kernel<DT>), dim3((unsigned)p.B), dim3(fin_threads(p.win)), 0, s, p);
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

// ---------------------------------------------------------------------------
// AsymSpec across model families (AsymSpec reading notes, the analysis of
// cross-family pairs): the drafter rows a, b live on the drafter vocabulary
// (V), the verifier row t on its own (Vt), and vmap[v] pairs verifier token
// v with a drafter token (string-identical tokens and paired specials) or
// is -1.  Generation is restricted to the paired tokens.
//
// Staged pass (rows of whole 16-byte vectors: Vd and Vt times the element
// size multiples of 16; the usual case):
//   Launch 1: the two-tensor row kernel over a, b (L_a, L_b, the JSD
//     partials); before leaving, its workgroups also build the inverse
//     alignment per part of the verifier row (xfam_invert_slice: xkey[p][d] =
//     i + 1 for each pair (v, d) with v the i-th token of part p, with a flag
//     when two such v share a drafter token).
//   Launch 2, xfam_staged_kernel: one 1024-thread workgroup per (row, part of
//     the verifier row, segment of the drafter row).  The part (at most
//     128 KiB) is copied into LDS behind one vector of -inf; the segment's a,
//     b and xkey[p] are streamed contiguously, and every drafter token reads
//     t at the LDS address of its key (the -inf slot when it has no pair in
//     the part).  So t, a and b are read once from memory, with no gathers.
//     Each thread keeps its maximum score and the lowest key (so verifier id)
//     reaching it.  Each workgroup also takes the online softmax statistics
//     of one share of its part.  Under a flagged map the pairs are met in
//     verifier order instead: v over the share, a and b gathered via vmap.
// General pass (any vocabulary sizes): launch 2 is xfam_verifier_kernel, one
// 256-thread workgroup per (row, 4096-token verifier chunk), a and b gathered
// through vmap; no keys are built.
// Launch 3, xfam_finalize_kernel: one workgroup per request; one wave per
// row combines both record sets and tests the draft (a verifier id) against
// the drafter's compressed-view probability of its pair, and one thread
// scans the request; after a staged pass its threads also clear the inverse
// alignment and the flag for the next call.
// ---------------------------------------------------------------------------

// Workgroup b runs on die b % 8 (round-robin dispatch); the chunks of one row
// go to workgroups of one die, so what they share of the row is fetched into
// one L2.  Returns false for the padding workgroups.
__device__ __forceinline__ bool xfam_item(const AsymParams &P, long long &row, int &chunk) {
    constexpr int kDies = 8;
    const long long b = blockIdx.x;
    const long long die = b % kDies, k = b / kDies;
    row = die + kDies * (k / P.vchunks);
    chunk = (int)(k % P.vchunks);
    return row < P.R;
}

// The running fused maximum of a thread and its lowest verifier id: a score
// replaces it when larger, or equal with a lower id (NaN scores never do).
struct FusedBest {
    float s;
    int v;
};
__device__ __forceinline__ void fused_take(FusedBest &fb, float sc, int v) {
    const bool take = (sc > fb.s) | ((sc == fb.s) & (v < fb.v)); // no short-circuit branch
    fb.s = take ? sc : fb.s;
    fb.v = take ? v : fb.v;
}

__device__ __forceinline__ uint32_t xword(const uint4 &w, int i) {
    return i == 0 ? w.x : i == 1 ? w.y : i == 2 ? w.z : w.w;
}

// The keys of one vector of logits: 16 bytes for bf16, 8 for fp32.
template <int DT> struct KeyVec;
template <> struct KeyVec<DT_BF16> {
    uint4 w;
    __device__ __forceinline__ void load(const uint16_t *keys, size_t q) {
        w = reinterpret_cast<const uint4 *>(keys)[q];
    }
    __device__ __forceinline__ uint32_t get(int e) const { return (xword(w, e >> 1) >> ((e & 1) * 16)) & 0xffffu; }
};
template <> struct KeyVec<DT_F32> {
    uint2 w;
    __device__ __forceinline__ void load(const uint16_t *keys, size_t q) {
        w = reinterpret_cast<const uint2 *>(keys)[q];
    }
    __device__ __forceinline__ uint32_t get(int e) const {
        return (((e >> 1) ? w.y : w.x) >> ((e & 1) * 16)) & 0xffffu;
    }
};

// The staged verifier value at LDS byte address `addr`.
template <int DT>
__device__ __forceinline__ float lds_at(const uint4 *lds, uint32_t addr) {
    const char *p = reinterpret_cast<const char *>(lds) + addr;
    if (DT == DT_BF16)
        return __uint_as_float((uint32_t)*reinterpret_cast<const uint16_t *>(p) << 16);
    return *reinterpret_cast<const float *>(p);
}

constexpr int kXlWaves = kXlThreads / 64;
// Vectors of the segment per thread per round.  One is fastest: at B = 64 a
// call took 0.132-0.134 ms with one, 0.135, 0.137 and 0.144 ms with two,
// three and four (the pass itself 51 us with one, 60 us with four).
constexpr int kXlUnroll = 1;

template <int DT>
__global__ __launch_bounds__(kXlThreads) void xfam_staged_kernel(AsymParams P) {
    constexpr int EPV = Elem<DT>::kPerVec;
    constexpr int U = kXlUnroll;
    // [0]: -inf (the slot of drafter tokens without a pair here), then the part
    __shared__ uint4 part[1 + kXlLdsVecs];
    __shared__ float lds_f[kXlWaves * 2];
    __shared__ double lds_d[kXlWaves];
    __shared__ int lds_i[kXlWaves];
    long long row;
    int chunk;
    if (!xfam_item(P, row, chunk))
        return;
    const int tid = threadIdx.x, wave = tid >> 6;
    const int pi = chunk % P.xparts, seg = chunk / P.xparts;
    const int plo = pi * P.xpartlen;
    const int plen = min(P.xpartlen, P.Vt - plo); // a multiple of EPV
    const float NEG_INF = -__builtin_inff();
    const bool drafter_order = ld_relaxed(P.xdup) == 0u;
    const size_t rv = (size_t)row * P.V / EPV;
    const uint4 *A4 = reinterpret_cast<const uint4 *>(P.a) + rv;
    const uint4 *B4 = reinterpret_cast<const uint4 *>(P.b) + rv;
    const uint16_t *keys = P.xkey + (size_t)pi * P.V;
    // LDS byte address of the token with key k: element k - 1 sits at
    // 16 + (k - 1)*size, and key 0 lands in the -inf vector
    constexpr uint32_t kEb = Elem<DT>::kBytes, kKeyBase = 16u - kEb;
    const int dlo = seg * P.xseglen, dhi = min(P.V, dlo + P.xseglen);
    const int q0 = dlo / EPV, q1 = dhi > dlo ? dhi / EPV : 0;

    // Vectors q + u*1024 of the segment; one past the end re-reads vector q,
    // which cannot change a maximum or a minimum.
    uint4 va[U], vb[U];
    KeyVec<DT> vk[U];
    auto load_round = [&](int q) {
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int qu = q + u * kXlThreads < q1 ? q + u * kXlThreads : q;
            va[u] = A4[qu];
            vb[u] = B4[qu];
            vk[u].load(keys, qu);
        }
    };

    // 1. the part into LDS, straight from memory, with the first round of the
    // segment already in flight
    if (tid == 0) {
        const uint32_t ni = DT == DT_BF16 ? 0xff80ff80u : 0xff800000u;
        part[0] = make_uint4(ni, ni, ni, ni);
    }
    {
        const uint4 *src = reinterpret_cast<const uint4 *>(P.tv) + ((size_t)row * P.Vt + plo) / EPV;
        const int nvec = plen / EPV;
#pragma unroll
        for (int j = 0; j < kXlLdsVecs / kXlThreads; ++j) {
            const int vi = j * kXlThreads + tid;
            if (vi < nvec)
                g2lds16(src + vi, part + 1 + j * kXlThreads + wave * 64);
        }
    }
    const int qs = q0 + tid;
    if (drafter_order && qs < q1)
        load_round(qs);
    __syncthreads();

    // 2. drafter order: the maximum fused score over the segment's pairs in
    // this part and the lowest key reaching it (keys grow with v).  A token
    // without a pair here reads the -inf slot, so its score is -inf or NaN,
    // and its key - 1 wraps to the largest value, so it never supplies the
    // index, not even when the maximum is -inf.
    float fm = NEG_INF;
    uint32_t fw = 0xffffffffu; // key - 1 of the best pair: its index in the part
    if (drafter_order) {
        for (int q = qs; q < q1; q += U * kXlThreads) {
            if (q != qs)
                load_round(q);
            float tv[U][EPV];
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < EPV; ++e)
                    tv[u][e] = lds_at<DT>(part, vk[u].get(e) * kEb + kKeyBase);
#pragma unroll
            for (int u = 0; u < U; ++u)
#pragma unroll
                for (int e = 0; e < EPV; ++e) {
                    const float sc = fused_score<kDeltaAMinusB>(widen<DT>(va[u], e), widen<DT>(vb[u], e), tv[u][e],
                                                                P.beta);
                    const uint32_t key = vk[u].get(e) - 1u;
                    const uint32_t lower = min(fw, key);
                    fw = sc == fm ? lower : fw;
                    fw = sc > fm ? key : fw;
                    fm = fmax_raw(fm, sc);
                }
        }
    }
    // 3. this segment's share of the part: L_t statistics (and, for a
    // flagged map, the pairs in verifier order)
    const int slo = min(plen, seg * P.xsharelen), shi = min(plen, slo + P.xsharelen);
    OnlineLse st;
    online_init(st);
    for (int vi = slo / EPV + tid; vi < shi / EPV; vi += kXlThreads) {
        const uint4 w = part[1 + vi];
        float x[EPV];
#pragma unroll
        for (int e = 0; e < EPV; ++e)
            x[e] = widen<DT>(w, e);
        online_group<EPV>(st, x);
    }
    FusedBest fb{NEG_INF, 0x7fffffff};
    if (!drafter_order) {
        const size_t arow = (size_t)row * P.V;
        for (int i = slo + tid; i < shi; i += kXlThreads) {
            const int d = P.vmap[plo + i];
            if (d >= 0 && d < P.V) {
                const float sc =
                    fused_score<kDeltaAMinusB>(load_scalar<DT>(P.a, arow + d), load_scalar<DT>(P.b, arow + d),
                                               lds_at<DT>(part, 16u + (uint32_t)i * Elem<DT>::kBytes), P.beta);
                fused_take(fb, sc, plo + i);
            }
        }
        fm = fb.s;
    }
    // 4. the workgroup's maximum, then its lowest verifier id
    float mx[2] = {st.c, fm};
    block_max<2, true, kXlWaves>(mx, lds_f);
    int fi = 0x7fffffff;
    if (fm == mx[1]) {
        if (!drafter_order)
            fi = fb.v;
        else if (fw != 0xffffffffu)
            fi = plo + (int)fw;
    }
    double S[1] = {rescale_to(st, mx[0])};
    block_sum_min<1, true, kXlWaves>(S, fi, lds_d, lds_i);
    if (tid == 0) {
        uint64_t *r = P.vrec + ((size_t)row * P.vchunks + chunk) * kVrecWords;
        r[0] = f64_bits(S[0]);
        r[1] = pack2(mx[0], mx[1]);
        r[2] = (uint64_t)(uint32_t)fi;
    }
}

template <int DT>
__global__ __launch_bounds__(kThreads) void xfam_verifier_kernel(AsymParams P) {
    __shared__ float lds_f[kWaves * 2];
    __shared__ double lds_d[kWaves];
    __shared__ int lds_i[kWaves];
    long long row;
    int chunk;
    if (!xfam_item(P, row, chunk))
        return;
    const int tid = threadIdx.x;
    const size_t trow = (size_t)row * (size_t)P.Vt, arow = (size_t)row * (size_t)P.V;
    const int v0 = chunk * kXfamChunk;
    const float NEG_INF = -__builtin_inff();
    // Branch-free so every load of a phase is in flight at once: out-of-range
    // elements read index 0 (always valid) and are masked afterwards.
    float x[kXfamEpt], xa[kXfamEpt], xb[kXfamEpt];
    int e[kXfamEpt];
    bool bad_map = false;
#pragma unroll
    for (int k = 0; k < kXfamEpt; ++k) { // element v0 + k*256 + tid: coalesced per wave
        const int v = v0 + k * kThreads + tid;
        const int vc = v < P.Vt ? v : 0;
        x[k] = load_scalar<DT>(P.tv, trow + vc);
        e[k] = P.vmap[vc];
    }
#pragma unroll
    for (int k = 0; k < kXfamEpt; ++k) {
        const bool in = v0 + k * kThreads + tid < P.Vt;
        bad_map |= in && (e[k] < -1 || e[k] >= P.V);
        if (!in || e[k] < 0 || e[k] >= P.V)
            e[k] = -1;
        if (!in)
            x[k] = NEG_INF;
        const int ec = e[k] >= 0 ? e[k] : 0;
        xa[k] = load_scalar<DT>(P.a, arow + ec);
        xb[k] = load_scalar<DT>(P.b, arow + ec);
    }
    FusedBest fb{NEG_INF, 0x7fffffff};
#pragma unroll
    for (int k = 0; k < kXfamEpt; ++k)
        if (e[k] >= 0)
            fused_take(fb, fused_score<kDeltaAMinusB>(xa[k], xb[k], x[k], P.beta), v0 + k * kThreads + tid);
    OnlineLse st;
    online_init(st);
    online_group<kXfamEpt>(st, x);
    float mx[2] = {st.c, fb.s};
    block_max<2>(mx, lds_f);
    int fi = (fb.s == mx[1]) ? fb.v : 0x7fffffff;
    double S[1] = {rescale_to(st, mx[0])};
    block_sum_min<1>(S, fi, lds_d, lds_i);
    if (tid == 0) {
        uint64_t *r = P.vrec + ((size_t)row * P.vchunks + chunk) * kVrecWords;
        r[0] = f64_bits(S[0]);
        r[1] = pack2(mx[0], mx[1]);
        r[2] = (uint64_t)(uint32_t)fi;
    }
    if (bad_map)
        set_dev_err(P.dev_err, 8);
}

// Row i of request bi, by one whole wave.
template <int DT>
__device__ __forceinline__ void xfam_finalize_row(const AsymParams &P, long long bi, int i, int lane,
                                                  uint32_t *sh_acc, int *sh_fi) {
    const long long row = bi * (P.K + 1) + i;
    // the draft (a verifier id), its pair and their logits, fetched by lane 0
    // while the records are combined
    int d = -1, e = -1;
    double td = 0.0, bd = 0.0;
    if (lane == 0 && i < P.K) {
        d = P.draft[bi * P.K + i];
        if (d >= 0 && d < P.Vt) {
            e = P.vmap[d];
            td = (double)load_scalar<DT>(P.tv, (size_t)row * (size_t)P.Vt + d);
            if (e >= 0 && e < P.V)
                bd = (double)load_scalar<DT>(P.b, (size_t)row * (size_t)P.V + e);
        }
    }
    // drafter side: L_b (log2 units) and the JSD partials
    const uint64_t *rec_row = P.rec + (size_t)row * P.Wmax * kRecWords;
    uint64_t w6[2] = {0, 0};
#pragma unroll
    for (int h = 0; h < 2; ++h)
        if (lane + 64 * h < P.W)
            w6[h] = ld_relaxed(rec_row + (size_t)(lane + 64 * h) * kRecWords + 6);
    double Lb2[1];
    team_lse<1>(rec_row, P.W, {1}, {3}, {true}, Lb2);
    double jsum = 0.0;
#pragma unroll
    for (int h = 0; h < 2; ++h)
        if (lane + 64 * h < P.W)
            jsum += as_f64(w6[h]);
    for (int w = lane + 128; w < P.W; w += 64) // teams wider than 128 members
        jsum += as_f64(ld_relaxed(rec_row + (size_t)w * kRecWords + 6));
    jsum = wave_sum(jsum);
    // verifier side: L_t and the fused token over the chunk records
    const uint64_t *vr = P.vrec + (size_t)row * P.vchunks * kVrecWords;
    double Lt2[1];
    team_lse<1>(vr, P.vchunks, {0}, {1}, {false}, Lt2, kVrecWords);
    float fbest = -__builtin_inff();
    for (int c = lane; c < P.vchunks; c += 64)
        fbest = fmaxf(fbest, unpack_hi(vr[(size_t)c * kVrecWords + 1]));
    fbest = wave_max(fbest);
    int fidx = 0x7fffffff;
    for (int c = lane; c < P.vchunks; c += 64)
        if (unpack_hi(vr[(size_t)c * kVrecWords + 1]) == fbest)
            fidx = min(fidx, (int)(uint32_t)vr[(size_t)c * kVrecWords + 2]);
    fidx = wave_min_int(fidx);
    if (fidx == 0x7fffffff)
        fidx = -1; // no verifier token is paired
    clear_row_exchange(P, row);
    for (int c = lane; c < P.vchunks; c += 64) { // the verifier records too (lane c read chunk c)
        uint64_t *r = P.vrec + ((size_t)row * P.vchunks + c) * kVrecWords;
#pragma unroll
        for (int k = 0; k < kVrecWords; ++k)
            r[k] = 0ull;
    }
    if (lane != 0)
        return;
    const double Lb = Lb2[0] * kLn2d, Lt = Lt2[0] * kLn2d;
    const double Dr = jsum;
    P.D[row] = (float)Dr;
    P.geff[row] = (float)((double)P.gamma * exp(-Dr));
    P.fused[row] = fidx;
    uint32_t acc = 0;
    if (i < P.K) {
        if (d < 0 || d >= P.Vt) {
            set_dev_err(P.dev_err, 1);
        } else {
            if (e >= 0 && e < P.V) { // an unpaired draft is rejected
                const double margin = (td - Lt) - (bd - Lb) - P.log_gamma + Dr;
                acc = margin > 0.0 ? 1u : 0u;
            }
        }
        P.accept[bi * P.K + i] = (uint8_t)acc;
    }
    sh_acc[i] = acc;
    sh_fi[i] = fidx;
}

template <int DT>
__global__ __launch_bounds__(kFinMaxThreads) void xfam_finalize_kernel(AsymParams P) {
    __shared__ uint32_t sh_acc[kMaxDrafts + 1];
    __shared__ int sh_fi[kMaxDrafts + 1];
    const int lane = threadIdx.x & 63;
    if (blockIdx.x == 0 && threadIdx.x == 0)
        P.ctl[0] = 0u; // ticket counter of the row kernel, for the next call
    // the inverse alignment and its flag, for the next call
    if (P.xparts > 0) {
        const long long n = (long long)xfam_key_words(P.xparts, P.V); // word n is the flag
        uint32_t *w = reinterpret_cast<uint32_t *>(P.xkey);
        for (long long i = (long long)blockIdx.x * blockDim.x + threadIdx.x; i <= n;
             i += (long long)gridDim.x * blockDim.x)
            w[i] = 0u;
    }
    const int Pn = P.K + 1;
    const long long bi = blockIdx.x;
    for (int i = (int)(threadIdx.x >> 6); i < Pn; i += (int)(blockDim.x >> 6))
        xfam_finalize_row<DT>(P, bi, i, lane, sh_acc, sh_fi);
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

// Workgroups of the verifier pass: 8 dies x (rows per die) x chunks.
inline long long xfam_verifier_grid(long long R, int chunks) { return 8 * ((R + 7) / 8) * (long long)chunks; }

template <int DT, int NV>
static hipError_t launch_x(const Plan &plan, const AsymParams &p, hipStream_t s, hipEvent_t after_rows) {
    // the row kernel's workgroups also build the staged pass's keys
    hipLaunchKernelGGL((asym_rows_kernel<DT, NV, kDeltaNone, kGateCda>), dim3(plan.grid), dim3(kThreads), 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    const unsigned vgrid = (unsigned)xfam_verifier_grid(p.R, p.vchunks);
    if (p.xparts > 0)
        hipLaunchKernelGGL((xfam_staged_kernel<DT>), dim3(vgrid), dim3(kXlThreads), 0, s, p);
    else
        hipLaunchKernelGGL((xfam_verifier_kernel<DT>), dim3(vgrid), dim3(kThreads), 0, s, p);
    e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (after_rows) {
        e = hipEventRecord(after_rows, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL((xfam_finalize_kernel<DT>), dim3((unsigned)p.B), dim3(fin_threads(p.K + 1)), 0, s, p);
    return hipGetLastError();
}

template <int DT>
static hipError_t launch_xnv(const Plan &plan, const AsymParams &p, hipStream_t s, hipEvent_t after_rows) {
    switch (plan.nv) {
    case 1: return launch_x<DT, 1>(plan, p, s, after_rows);
    case 2: return launch_x<DT, 2>(plan, p, s, after_rows);
    case 4: return launch_x<DT, 4>(plan, p, s, after_rows);
    case 8: return launch_x<DT, 8>(plan, p, s, after_rows);
    }
    return hipErrorInvalidValue;
}

hipError_t launch_xfam(int dt, const Plan &plan, const AsymParams &p, hipStream_t s, hipEvent_t after_rows) {
    return dt == DT_BF16 ? launch_xnv<DT_BF16>(plan, p, s, after_rows) : launch_xnv<DT_F32>(plan, p, s, after_rows);
}

} // namespace vwl
