// AsymSpec from hidden states: the LM heads' products formed on the matrix
// cores with the row statistics in their epilogue (the step before the
// AsymSpec pass on its pages: the drafter's head turns the full- and
// compressed-context hidden states into a and b, the verifier's head turns
// its hidden state into t).
//
//   a = h_a W_d^T, b = h_b W_d^T   (one drafter head, two views)
//   t = h_t W_t^T
//
// Launch 1, lmhead_kernel<1, STORE, G>: each workgroup owns 64 G rows (G
// groups of 4 waves: one group up to 128 rows, three past that) and a range
// of the vocabulary, walked in tiles of 128 tokens.  Per tile each group's
// 4 waves form a [64 x 128] block of a, b (all groups sharing each W_d
// tile) and then of t with bf16 MFMA 16x16x32 (fp32 accumulation), staged
// through LDS in 64-wide k blocks (with three groups in two buffers, the
// next block's loads in flight during the current one); the epilogue folds
// the block into per-row online statistics of a, b, t (integer references,
// as in the row kernel) and the fused maximum t + beta*(a - b) with its
// lowest index, and, with a workspace that holds them, stores the (a, b)
// pairs as fp32 for the JSD.  One record per (row, range), in the row
// kernel's record layout.
// Launch 2, lmhead_combine_kernel: per row, L_a, L_b, L_t and the fused
// token from the records, and the draft's logits as fp64 dot products.
// Launch 3, the JSD terms against L_a, L_b: lmhead_jsd_kernel over the stored
// pairs, one partial sum per (row, 4096-token chunk); or, with no pair
// storage (no logit is then ever written), lmhead_kernel<2, false, 1>: a
// and b formed again by the same arithmetic (the same bits), one partial per
// (row, range).
// Launch 4, lmhead_finalize_kernel: D, the threshold, the test and the scan.
#include "asym_kernels.hpp"

namespace vwl {

typedef __bf16 bf16x8_t __attribute__((ext_vector_type(8)));
typedef float f32x4_t __attribute__((ext_vector_type(4)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));

constexpr int kLmRows = kLmRowTile; // rows per group of 4 waves
constexpr int kLmM = kLmRows / 16;   // MFMA row blocks of 16
constexpr int kLmCols = 128; // vocabulary per tile (32 per wave, 2 MFMA column blocks)
constexpr int kLmKB = 64;    // k per LDS stage (2 MFMA k-steps of 32)
// A workgroup is G groups of 4 waves over 64 G rows; the groups share each
// head tile.  Waves issuing the head tile's staging loads:
template <int G>
constexpr int lm_w_waves() { return G == 1 ? 4 : 8; }

// One stage: [rows][8 chunks of 8 bf16]; chunk c of row r sits in slot
// c ^ (r & 7), so the 16 rows an MFMA operand read touches spread over the
// banks.
template <int G>
struct LmStage {
    uint4 a[G * kLmRows * 8];
    uint4 b[G * kLmRows * 8];
    uint4 w[kLmCols * 8];
};

__device__ __forceinline__ int lm_slot(int r, int c) { return r * 8 + (c ^ (r & 7)); }

// Staging of rows [row0, row0 + NR) (rows past max_row repeat it) of a
// row-major bf16 matrix with H columns, one 64-wide k block at a time.
// Instruction j of the block (issued by wave j mod 4) fills LDS slots
// 64 j .. 64 j + 63, so each instruction reads 8 whole 128-byte row pieces.
// The lane's byte offsets from the block's base are the same for every k
// block of a tile, so they are formed once per tile; per block the loads
// are a scalar base plus those offsets, with no vector arithmetic.
template <int NR, int NW>
struct LmLoads {
    static constexpr int kN = NR * 8 / 64 / NW; // instructions per issuing wave
    static_assert(NR * 8 % (64 * NW) == 0, "every issuing wave issues the same number of stage loads");
    uint32_t off[kN]; // lane byte offsets from the block base
    uint32_t lds[kN]; // LDS destinations (wave-uniform)
};

template <int NR, int NW>
__device__ __forceinline__ void lm_loads(LmLoads<NR, NW> &L, uint4 *dst, long long row0, long long max_row, int H) {
    const int lane = threadIdx.x & 63;
    const int wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) % NW; // non-issuing waves: unused
#pragma unroll
    for (int i = 0; i < LmLoads<NR, NW>::kN; ++i) {
        const int j = wave + i * NW;
        const int p = j * 64 + lane;
        const int r = p >> 3, slot = p & 7;
        const int c = slot ^ (r & 7);
        const long long row = row0 + r > max_row ? max_row : row0 + r;
        L.off[i] = (uint32_t)(((row - row0) * (long long)H + 8 * c) * 2);
        L.lds[i] = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(dst + j * 64));
    }
}

// Issue one k block: `base` is the wave-uniform address of (row0, k0).  The
// loads are inline assembly (an SGPR base plus the lane's offset; `s_nop 4`
// gives the wait states the hardware needs after M0 or the base is
// written), so the compiler does not track them: lm_gemm waits for them
// explicitly before its barrier.
template <int NR, int NW>
__device__ __forceinline__ void lm_issue(const LmLoads<NR, NW> &L, const uint16_t *base) {
    if (__builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) >= NW)
        return;
#pragma unroll
    for (int i = 0; i < LmLoads<NR, NW>::kN; ++i)
        asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(L.off[i]), "s"(base), "{m0}"(L.lds[i])
                     : "memory");
}

__device__ __forceinline__ bf16x8_t lm_frag(const uint4 *tile, int r, int c) {
    const uint4 v = tile[lm_slot(r, c)];
    bf16x8_t f;
    __builtin_memcpy(&f, &v, 16);
    return f;
}

// All-reductions over the 16 lanes of a DPP row (the lanes that share rows
// in the MFMA 16x16 accumulator layout).
__device__ __forceinline__ float row16_max(float x) {
    x = fmaxf(x, __int_as_float(dpp_i<kDppXor1>(__float_as_int(x))));
    x = fmaxf(x, __int_as_float(dpp_i<kDppXor2>(__float_as_int(x))));
    x = fmaxf(x, __int_as_float(dpp_i<kDppHalfMirror>(__float_as_int(x))));
    return fmaxf(x, __int_as_float(dpp_i<kDppMirror>(__float_as_int(x))));
}
__device__ __forceinline__ float row16_sum(float x) {
    x += __int_as_float(dpp_i<kDppXor1>(__float_as_int(x)));
    x += __int_as_float(dpp_i<kDppXor2>(__float_as_int(x)));
    x += __int_as_float(dpp_i<kDppHalfMirror>(__float_as_int(x)));
    return x + __int_as_float(dpp_i<kDppMirror>(__float_as_int(x)));
}
__device__ __forceinline__ int row16_min_int(int x) {
    x = min(x, dpp_i<kDppXor1>(x));
    x = min(x, dpp_i<kDppXor2>(x));
    x = min(x, dpp_i<kDppHalfMirror>(x));
    return min(x, dpp_i<kDppMirror>(x));
}

// The [64 G x 128] block of one head for one or two sets of hidden states
// (TWO: h0 and h1 share the head tile), accumulated over k in [0, H); each
// wave forms [64 x 32] of it (group wave / 4, columns of wave % 4).  With
// NS = 2 staging buffers the loads of k block i + 1 are in flight while the
// waves work on block i (barriers without a wait for global loads, and an
// explicit wait for all but the block just issued).
template <bool TWO, int G, int NS>
__device__ __forceinline__ void lm_gemm(LmStage<G> (&st)[NS], const uint16_t *h0, const uint16_t *h1,
                                        const uint16_t *W, long long row0, long long R, long long vt0, int V, int H,
                                        f32x4_t (&acc0)[kLmM][2], f32x4_t (&acc1)[kLmM][2]) {
    using LA = LmLoads<G * kLmRows, 4 * G>;
    using LW = LmLoads<kLmCols, lm_w_waves<G>()>;
    const int lane = threadIdx.x & 63;
    const int wq = (threadIdx.x >> 6) & 3;        // the wave's 32 columns
    const int gr = kLmRows * (threadIdx.x >> 8); // the wave's group's first row
#pragma unroll
    for (int m = 0; m < kLmM; ++m)
#pragma unroll
        for (int n = 0; n < 2; ++n) {
            acc0[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
            acc1[m][n] = f32x4_t{0.f, 0.f, 0.f, 0.f};
        }
    LA la;
    LW lw;
    lm_loads(la, st[0].a, row0, R - 1, H);
    lm_loads(lw, st[0].w, vt0, V - 1, H);
    const uint32_t lds_b = (uint32_t)(reinterpret_cast<uintptr_t>(st[0].b) - reinterpret_cast<uintptr_t>(st[0].a));
    const uint32_t lds_s =
        NS == 2 ? (uint32_t)(reinterpret_cast<uintptr_t>(&st[NS - 1]) - reinterpret_cast<uintptr_t>(&st[0])) : 0u;
    const uint16_t *pa = h0 + row0 * H, *pw = W + vt0 * H;
    const uint16_t *pb = TWO ? h1 + row0 * H : nullptr;
    auto issue = [&](int k0, int buf) {
        LA l1 = la;
        LW l2 = lw;
        if (buf) {
#pragma unroll
            for (int i = 0; i < LA::kN; ++i)
                l1.lds[i] += lds_s;
#pragma unroll
            for (int i = 0; i < LW::kN; ++i)
                l2.lds[i] += lds_s;
        }
        lm_issue(l1, pa + k0);
        if (TWO) {
            LA l3 = l1; // same rows and slots, the second view's LDS tile
#pragma unroll
            for (int i = 0; i < LA::kN; ++i)
                l3.lds[i] += lds_b;
            lm_issue(l3, pb + k0);
        }
        lm_issue(l2, pw + k0);
    };
    auto compute = [&](const LmStage<G> &sg) {
#pragma unroll 1
        for (int s = 0; s < kLmKB / 32; ++s) {
            const int c = 4 * s + (lane >> 4);
            bf16x8_t fw[2];
#pragma unroll
            for (int n = 0; n < 2; ++n)
                fw[n] = lm_frag(sg.w, 32 * wq + 16 * n + (lane & 15), c);
#pragma unroll
            for (int m = 0; m < kLmM; ++m) {
                const bf16x8_t f0 = lm_frag(sg.a, gr + 16 * m + (lane & 15), c);
#pragma unroll
                for (int n = 0; n < 2; ++n)
                    acc0[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f0, fw[n], acc0[m][n], 0, 0, 0);
                if (TWO) {
                    const bf16x8_t f1 = lm_frag(sg.b, gr + 16 * m + (lane & 15), c);
#pragma unroll
                    for (int n = 0; n < 2; ++n)
                        acc1[m][n] = __builtin_amdgcn_mfma_f32_16x16x32_bf16(f1, fw[n], acc1[m][n], 0, 0, 0);
                }
            }
        }
    };
    if constexpr (NS == 1) {
        for (int k0 = 0; k0 < H; k0 += kLmKB) {
            __syncthreads(); // every wave is done with the previous stage
            issue(k0, 0);
            __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            __syncthreads();
            compute(st[0]);
        }
    } else {
        // this wave's staging loads per block: h (one or two views) and, for
        // the waves that stage it, the head tile
        const bool w_wave = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) < lm_w_waves<G>();
        const int n_blk = LA::kN * (TWO ? 2 : 1) + (w_wave ? LW::kN : 0);
        __syncthreads(); // the buffers' previous readers are done
        issue(0, 0);
        int buf = 0;
        for (int k0 = 0; k0 < H; k0 += kLmKB) {
            const bool more = k0 + kLmKB < H;
            if (more) {
                issue(k0 + kLmKB, buf ^ 1);
                // all but the block just issued (loads complete in order)
                if (n_blk == 6)
                    __asm__ volatile("s_waitcnt vmcnt(6)" ::: "memory");
                else if (n_blk == 4)
                    __asm__ volatile("s_waitcnt vmcnt(4)" ::: "memory");
                else if (n_blk == 2)
                    __asm__ volatile("s_waitcnt vmcnt(2)" ::: "memory");
                else
                    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            } else {
                __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
            }
            lds_barrier(); // every wave's loads of this buffer have landed
            compute(st[buf]);
            lds_barrier(); // every wave is done with this buffer before its refill
            buf ^= 1;
        }
    }
}

// Row of accumulator slot (m, j) in the workgroup's 64 G rows, and column of
// block n in the tile's 128.
__device__ __forceinline__ int lm_row(int m, int j) {
    return kLmRows * (threadIdx.x >> 8) + 16 * m + 4 * ((threadIdx.x & 63) >> 4) + j;
}
__device__ __forceinline__ int lm_col(int n) { return 32 * ((threadIdx.x >> 6) & 3) + 16 * n + (threadIdx.x & 15); }

// The waves' partials of a tile: a's and b's statistics, then t's and the
// fused maxima with their columns.
// [column quarter][row]: the 4 waves of a row's group.
template <int G>
struct LmScratch {
    float ref0[4][G * kLmRows]; // a, then t
    float sum0[4][G * kLmRows];
    float ref1[4][G * kLmRows]; // b, then the fused maxima
    union {
        float sum1[4][G * kLmRows]; // b
        int fi[4][G * kLmRows];     // the fused maxima's columns
    };
};
// Running per-row state of the workgroup's rows across its tiles (in LDS,
// so that no register holds it across the k loops): the statistics of the
// first pass, or the JSD sum of the recomputing pass.
template <int G>
struct LmRun {
    double s[3][G * kLmRows];
    float c[3][G * kLmRows];
    float fm[G * kLmRows];
    int fi[G * kLmRows];
};
// Row constants of the recomputing pass: L_a, L_b (log2 units) and their
// difference in nats as a float pair.
template <int G>
struct LmRowC {
    float la[G * kLmRows], lb[G * kLmRows], dh[G * kLmRows], dlo[G * kLmRows];
};
// Merge a partial (reference c, sum s) into a running fp64 state.
__device__ __forceinline__ void lm_merge(float &run_c, double &run_s, float c, double s) {
    const float C = fmaxf(run_c, c);
    run_s = scale_pow2(run_s, run_c - C) + scale_pow2(s, c - C);
    run_c = C;
}

// Fold the waves' partials of tensor k into its running state (one thread
// per row), the waves in column order.
template <int G>
__device__ __forceinline__ void lm_fold_one(LmRun<G> &run, int k, const float (&ref)[4][G * kLmRows],
                                            const float (&sum)[4][G * kLmRows]) {
    const int tid = threadIdx.x;
    float c = run.c[k][tid];
    double sm = run.s[k][tid];
#pragma unroll
    for (int w = 0; w < 4; ++w)
        lm_merge(c, sm, ref[w][tid], (double)sum[w][tid]);
    run.c[k][tid] = c;
    run.s[k][tid] = sm;
}
// The tile's partials into the running state: threads 0..63, one row each.
// AB: a and b (tensors 0 and 1); else t (tensor 2) and the fused maxima (a
// strict > keeps the lowest index).
template <bool AB, int G>
__device__ __forceinline__ void lm_fold(LmRun<G> &run, const LmScratch<G> &sc, long long vt0) {
    const int tid = threadIdx.x;
    if (tid >= G * kLmRows)
        return;
    if (AB) {
        lm_fold_one<G>(run, 0, sc.ref0, sc.sum0);
        lm_fold_one<G>(run, 1, sc.ref1, sc.sum1);
    } else {
        lm_fold_one<G>(run, 2, sc.ref0, sc.sum0);
        float fm = run.fm[tid];
        int fi = run.fi[tid];
#pragma unroll
        for (int w = 0; w < 4; ++w) {
            if (sc.ref1[w][tid] > fm) {
                fm = sc.ref1[w][tid];
                fi = (int)vt0 + sc.fi[w][tid];
            }
        }
        run.fm[tid] = fm;
        run.fi[tid] = fi;
    }
}

// Per-row statistics of one tensor's block held as accumulators, written to
// the wave's scratch: for each of the lane's rows (m, j) the integer
// reference and the fp32 sum of 2^(x*log2e - ref) over the wave's 32 columns
// (identical in the 16 lanes of a DPP row; lane 0 of the row writes).
// Invalid columns count as -inf.
template <int G>
__device__ __forceinline__ void lm_tile_stats(float (&ref)[4][G * kLmRows], float (&sum)[4][G * kLmRows],
                                              const f32x4_t (&x)[kLmM][2], const bool (&cv)[2]) {
    const float NEG_INF = -__builtin_inff();
    const int wave = (threadIdx.x >> 6) & 3;
#pragma unroll
    for (int m = 0; m < kLmM; ++m)
#pragma unroll
        for (int j = 0; j < 4; ++j) {
            const float x0 = cv[0] ? x[m][0][j] : NEG_INF, x1 = cv[1] ? x[m][1][j] : NEG_INF;
            const float mx = row16_max(fmaxf(x0, x1));
            const float c = __builtin_ceilf(fmaxf(mx, -1e30f) * kLog2e);
            const float sm = row16_sum(__builtin_amdgcn_exp2f(__fmaf_rn(x0, kLog2e, -c)) +
                                       __builtin_amdgcn_exp2f(__fmaf_rn(x1, kLog2e, -c)));
            if ((threadIdx.x & 15) == 0) {
                ref[wave][lm_row(m, j)] = c;
                sum[wave][lm_row(m, j)] = sm;
            }
        }
}


// PASS 1: the statistics of a, b, t and the fused maximum; with STORE the
// (a, b) pairs are also written for the JSD pass.  PASS 2 (the path with no
// pair storage): a and b formed again by the same code, so with the same
// bits, and the JSD terms against L_a, L_b summed into one partial per (row,
// range).
template <int PASS, bool STORE, int G>
__global__ __launch_bounds__(kThreads * G, (G == 1 ? 3 : 1)) void lmhead_kernel(LmheadParams P) {
    constexpr int kRowsWg = G * kLmRows;
    constexpr int NS = G == 1 ? 1 : 2; // staging buffers
    // the staging buffers first, at LDS address 0: the staging loads take
    // their LDS address from M0
    __shared__ struct {
        LmStage<G> st[NS];
        LmScratch<G> sc;
        LmRun<G> run;
        LmRowC<G> rowc;
    } sh;
    LmStage<G> (&st)[NS] = sh.st;
    LmScratch<G> &sc = sh.sc;
    LmRun<G> &run = sh.run;
    LmRowC<G> &rowc = sh.rowc;
    const int tid = threadIdx.x, lane = tid & 63, wave = (tid >> 6) & 3;
    // workgroup b runs on die b % 8: the row tiles of one vocabulary range
    // share a die, so its head tiles come from one L2
    const long long b = blockIdx.x;
    const long long q = b / 8;
    const int rtile = (int)(q % P.RT);
    const int s = (int)(8 * (q / P.RT) + b % 8);
    if (s >= P.S)
        return;
    const long long row0 = (long long)rtile * kRowsWg;
    const long long v_begin = (long long)s * P.range;
    const long long v_end = min((long long)P.V, v_begin + P.range);
    const float NEG = -3.0e38f;

    // running per-row state in LDS (one thread per row, row = tid)
    if (tid < kRowsWg) {
#pragma unroll
        for (int k = 0; k < 3; ++k) {
            run.c[k][tid] = NEG;
            run.s[k][tid] = 0.0;
        }
        run.fm[tid] = -__builtin_inff();
        run.fi[tid] = 0x7fffffff;
        if (PASS == 2) {
            const long long row = min(row0 + tid, P.R - 1);
            const double La2 = P.rowstat[row * kLmStat + 0], Lb2 = P.rowstat[row * kLmStat + 1];
            const double dl = (La2 - Lb2) * kLn2d;
            rowc.la[tid] = (float)La2;
            rowc.lb[tid] = (float)Lb2;
            rowc.dh[tid] = (float)dl;
            rowc.dlo[tid] = (float)(dl - (double)(float)dl);
        }
    }

    for (long long vt0 = v_begin; vt0 < v_end; vt0 += kLmCols) {
        bool cv[2];
#pragma unroll
        for (int n = 0; n < 2; ++n)
            cv[n] = vt0 + lm_col(n) < v_end;
        f32x4_t xa[kLmM][2], xb[kLmM][2];
        lm_gemm<true, G, NS>(st, P.ha, P.hb, P.Wd, row0, P.R, vt0, P.V, P.Hd, xa, xb);
        if (PASS == 2) {
            // JSD terms of the block against the row's log-sum-exps
#pragma unroll
            for (int m = 0; m < kLmM; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    const int r = lm_row(m, j);
                    const float la_c = rowc.la[r], lb_c = rowc.lb[r], dh = rowc.dh[r], dlo = rowc.dlo[r];
                    float J = 0.f;
#pragma unroll
                    for (int n = 0; n < 2; ++n) {
                        if (cv[n]) {
                            const float a = xa[m][n][j], bb = xb[m][n][j];
                            J += jsd_term(__fmaf_rn(a, kLog2e, -la_c), __fmaf_rn(bb, kLog2e, -lb_c),
                                          ((a - bb) - dh) - dlo);
                        }
                    }
                    J = row16_sum(J);
                    if ((lane & 15) == 0)
                        sc.sum0[wave][r] = J;
                }
            __syncthreads();
            if (tid < kRowsWg) { // the waves in column order
                double t = run.s[0][tid];
#pragma unroll
                for (int w = 0; w < 4; ++w)
                    t += (double)sc.sum0[w][tid];
                run.s[0][tid] = t;
            }
            continue;
        }
        // with STORE, the pairs for the JSD pass, streamed (read once, by
        // the next launch but one): lg has a row for every row of the tile
        // and a column for every column of the tile, so the stores need no
        // guard (the pairs past R or V are never read).  The row stride is
        // re-read opaquely per tile, so the 16 row offsets are formed here
        // rather than held in registers across the loop.
        if (STORE) {
            long long lgs = P.lgs;
            asm volatile("" : "+s"(lgs));
            f32x2_t *q = reinterpret_cast<f32x2_t *>(P.lg) + (row0 + lm_row(0, 0)) * lgs + vt0 + lm_col(0);
#pragma unroll
            for (int m = 0; m < kLmM; ++m)
#pragma unroll
                for (int j = 0; j < 4; ++j) {
                    f32x2_t *qr = q + (long long)(16 * m + j) * lgs;
                    __builtin_nontemporal_store(f32x2_t{xa[m][0][j], xb[m][0][j]}, qr);
                    __builtin_nontemporal_store(f32x2_t{xa[m][1][j], xb[m][1][j]}, qr + 16);
                }
        }
        lm_tile_stats<G>(sc.ref0, sc.sum0, xa, cv);
        lm_tile_stats<G>(sc.ref1, sc.sum1, xb, cv);
#pragma unroll
        for (int m = 0; m < kLmM; ++m)
#pragma unroll
            for (int n = 0; n < 2; ++n)
                xa[m][n] = xa[m][n] - xb[m][n];
        __syncthreads();
        lm_fold<true, G>(run, sc, vt0);
        f32x4_t xt[kLmM][2], unused[kLmM][2];
        lm_gemm<false, G, NS>(st, P.ht, nullptr, P.Wt, row0, P.R, vt0, P.V, P.Ht, xt, unused);
        lm_tile_stats<G>(sc.ref0, sc.sum0, xt, cv);
#pragma unroll
        for (int m = 0; m < kLmM; ++m)
#pragma unroll
            for (int j = 0; j < 4; ++j) {
                // fused score t + beta*(a - b), its maximum and lowest column
                const float f0 = cv[0] ? __fmaf_rn(P.beta, xa[m][0][j], xt[m][0][j]) : -__builtin_inff();
                const float f1 = cv[1] ? __fmaf_rn(P.beta, xa[m][1][j], xt[m][1][j]) : -__builtin_inff();
                const bool second = f1 > f0;
                const float fb = second ? f1 : f0;
                const int col = lm_col(second ? 1 : 0);
                const float fm = row16_max(fb);
                const int fi = row16_min_int((fb == fm && (cv[0] || cv[1])) ? col : 0x7fffffff);
                if ((lane & 15) == 0) {
                    sc.ref1[wave][lm_row(m, j)] = fm;
                    sc.fi[wave][lm_row(m, j)] = fi;
                }
            }
        __syncthreads();
        lm_fold<false, G>(run, sc, vt0);
    }
    const long long row = row0 + tid;
    if (PASS == 2) {
        if (tid < kRowsWg && row < P.R)
            P.jpart[row * P.jc + s] = run.s[0][tid];
        return;
    }
    if (tid < kRowsWg && row < P.R) {
        uint64_t *rec = P.rec + ((size_t)row * P.S + s) * kRecWords;
        rec[0] = f64_bits(run.s[0][tid]);
        rec[1] = f64_bits(run.s[1][tid]);
        rec[2] = f64_bits(run.s[2][tid]);
        rec[3] = pack2(run.c[0][tid], run.c[1][tid]);
        rec[4] = pack2(run.c[2][tid], run.fm[tid]);
        rec[5] = (uint64_t)(uint32_t)run.fi[tid];
    }
}

// fp64 dot product of two bf16 rows of length H (one whole wave).
// Five 512-element blocks per round are loaded together (a block past the
// end re-reads the lane's first vector and is skipped), then summed in
// element order.
__device__ __forceinline__ double lm_dot(const uint16_t *x, const uint16_t *y, int H) {
    constexpr int U = 5;
    const int k_lane = (threadIdx.x & 63) * 8;
    double acc = 0.0;
    for (int k0 = k_lane; k0 < H; k0 += 64 * 8 * U) {
        uint4 vx[U], vy[U];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int k = k0 + 64 * 8 * u < H ? k0 + 64 * 8 * u : k_lane;
            vx[u] = *reinterpret_cast<const uint4 *>(x + k);
            vy[u] = *reinterpret_cast<const uint4 *>(y + k);
        }
#pragma unroll
        for (int u = 0; u < U; ++u)
            if (k0 + 64 * 8 * u < H)
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    acc += (double)widen<DT_BF16>(vx[u], e) * (double)widen<DT_BF16>(vy[u], e);
    }
    return wave_sum(acc);
}

// Launch 2: one workgroup per row.  L_a, L_b, L_t (log2 units) and the fused
// token from the row's records (each thread folds every 256th record,
// five at a time, then the workgroup merges the threads' states), and for a
// draft row the draft's logits t_d, b_d as fp64 dot products of the stored
// values.  rowstat[row] = {L_a, L_b, L_t, fused token, t_d, b_d}.
__global__ __launch_bounds__(kThreads) void lmhead_combine_kernel(LmheadParams P) {
    __shared__ float shf[kWaves * 4];
    __shared__ double shd[kWaves * 3];
    __shared__ int shi[kWaves];
    const long long row = blockIdx.x;
    const uint64_t *rec_row = P.rec + (size_t)row * P.S * kRecWords;
    const float NEG = -3.0e38f;
    float C[3] = {NEG, NEG, NEG};
    double sum[3] = {0.0, 0.0, 0.0};
    float fbest = -__builtin_inff();
    int fidx = 0x7fffffff;
    constexpr int U = 5;
    for (int w0 = threadIdx.x; w0 < P.S; w0 += kThreads * U) {
        uint64_t r[U][6];
#pragma unroll
        for (int u = 0; u < U; ++u) {
            const int w = w0 + kThreads * u < P.S ? w0 + kThreads * u : w0;
#pragma unroll
            for (int k = 0; k < 6; ++k)
                r[u][k] = rec_row[(size_t)w * kRecWords + k];
        }
#pragma unroll
        for (int u = 0; u < U; ++u) {
            if (w0 + kThreads * u < P.S) {
                lm_merge(C[0], sum[0], unpack_lo(r[u][3]), as_f64(r[u][0]));
                lm_merge(C[1], sum[1], unpack_hi(r[u][3]), as_f64(r[u][1]));
                lm_merge(C[2], sum[2], unpack_lo(r[u][4]), as_f64(r[u][2]));
                const float fm = unpack_hi(r[u][4]);
                const int fi = (int)(uint32_t)r[u][5];
                fidx = fm > fbest ? fi : (fm == fbest ? min(fidx, fi) : fidx);
                fbest = fmaxf(fbest, fm);
            }
        }
    }
    float m[4] = {C[0], C[1], C[2], fbest};
    block_max<4>(m, shf);
    double t[3];
#pragma unroll
    for (int k = 0; k < 3; ++k)
        t[k] = scale_pow2(sum[k], C[k] - m[k]);
    int imin = fbest == m[3] ? fidx : 0x7fffffff;
    block_sum_min<3>(t, imin, shd, shi);
    const int wave = threadIdx.x >> 6;
    double *rs = P.rowstat + row * kLmStat;
    if (threadIdx.x == 0) {
        rs[0] = (double)m[0] + log2(t[0]);
        rs[1] = (double)m[1] + log2(t[1]);
        rs[2] = (double)m[2] + log2(t[2]);
        rs[3] = (double)imin;
    }
    const long long bi = row / (P.K + 1);
    const int i = (int)(row % (P.K + 1));
    if (i < P.K && wave < 2) {
        const int d = P.draft[bi * P.K + i];
        if (d >= 0 && d < P.V) { // the draft's logits, exactly products of the stored values
            const double x = wave == 0 ? lm_dot(P.ht + (size_t)row * P.Ht, P.Wt + (size_t)d * P.Ht, P.Ht)
                                       : lm_dot(P.hb + (size_t)row * P.Hd, P.Wd + (size_t)d * P.Hd, P.Hd);
            if ((threadIdx.x & 63) == 0)
                rs[4 + wave] = x;
        }
    }
}

// Row i of request bi from its statistics and JSD partials, by one whole
// wave; lane 0 writes the row's outputs.
__device__ __forceinline__ void lmhead_finalize_row(const LmheadParams &P, long long bi, int i, int lane,
                                                    uint32_t *sh_acc, int *sh_fi) {
    const long long row = bi * (P.K + 1) + i;
    double jsum = 0.0;
    for (int c = lane; c < P.jc; c += 64)
        jsum += P.jpart[row * P.jc + c];
    jsum = wave_sum(jsum);
    if (lane != 0)
        return;
    const double *rs = P.rowstat + row * kLmStat;
    const int fidx = (int)rs[3];
    const double Dr = -0.5 * kLn2d * jsum;
    P.D[row] = (float)Dr;
    P.geff[row] = (float)((double)P.gamma * exp(-Dr));
    P.fused[row] = fidx;
    uint32_t acc = 0;
    if (i < P.K) {
        const int d = P.draft[bi * P.K + i];
        if (d < 0 || d >= P.V) {
            set_dev_err(P.dev_err, 1);
        } else {
            const double Lb = rs[1] * kLn2d, Lt = rs[2] * kLn2d;
            const double margin = (rs[4] - Lt) - (rs[5] - Lb) - P.log_gamma + Dr;
            acc = margin > 0.0 ? 1u : 0u;
        }
        P.accept[bi * P.K + i] = (uint8_t)acc;
    }
    sh_acc[i] = acc;
    sh_fi[i] = fidx;
}

// Launch 3: the JSD terms of one row's stored pairs in [4096 c, 4096 c + 4096)
// against the row's log-sum-exps, workgroup (row, c).  Each load instruction
// reads 4 KB of consecutive pairs (streamed: they are read once); a thread
// sums its 16 terms in fp32, the workgroup in fp64.
__global__ __launch_bounds__(kThreads) void lmhead_jsd_kernel(LmheadParams P) {
    __shared__ double sh[kWaves];
    const long long row = blockIdx.x / P.jc;
    const int c = (int)(blockIdx.x % P.jc);
    const double La2 = P.rowstat[row * kLmStat + 0], Lb2 = P.rowstat[row * kLmStat + 1];
    const double dl = (La2 - Lb2) * kLn2d;
    const float la = (float)La2, lb = (float)Lb2, dh = (float)dl, dlo = (float)(dl - (double)dh);
    // two pairs per 16-byte vector; a vector starting below V lies inside the
    // row, whose stride is even
    typedef float f4v __attribute__((ext_vector_type(4)));
    const f4v *src = reinterpret_cast<const f4v *>(P.lg + (size_t)row * P.lgs * 2);
    const long long e0 = (long long)c * kLmJsdChunk + 2 * threadIdx.x;
    constexpr int kVec = kLmJsdPairs / 2;
    f4v v[kVec];
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
        const long long e = e0 + 2LL * kThreads * i;
        v[i] = e < P.V ? __builtin_nontemporal_load(src + (e >> 1)) : f4v{0.f, 0.f, 0.f, 0.f};
    }
    float J = 0.f;
#pragma unroll
    for (int i = 0; i < kVec; ++i) {
        const long long e = e0 + 2LL * kThreads * i;
        if (e < P.V)
            J += jsd_term(__fmaf_rn(v[i].x, kLog2e, -la), __fmaf_rn(v[i].y, kLog2e, -lb), ((v[i].x - v[i].y) - dh) - dlo);
        if (e + 1 < P.V)
            J += jsd_term(__fmaf_rn(v[i].z, kLog2e, -la), __fmaf_rn(v[i].w, kLog2e, -lb), ((v[i].z - v[i].w) - dh) - dlo);
    }
    const double w = wave_sum((double)J);
    if ((threadIdx.x & 63) == 0)
        sh[threadIdx.x >> 6] = w;
    __syncthreads();
    if (threadIdx.x == 0) {
        double t = 0.0;
#pragma unroll
        for (int k = 0; k < kWaves; ++k)
            t += sh[k];
        P.jpart[row * P.jc + c] = t;
    }
}

// Launch 4: one workgroup per request, one wave per row (up to 16 waves; wave
// w takes rows w, w + 16, ...), then one thread scans the accept flags.
__global__ __launch_bounds__(kFinMaxThreads) void lmhead_finalize_kernel(LmheadParams P) {
    __shared__ uint32_t sh_acc[kMaxDrafts + 1];
    __shared__ int sh_fi[kMaxDrafts + 1];
    const long long bi = blockIdx.x;
    for (int i = (int)(threadIdx.x >> 6); i < P.K + 1; i += (int)(blockDim.x >> 6))
        lmhead_finalize_row(P, bi, i, threadIdx.x & 63, sh_acc, sh_fi);
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

int lmhead_blocks_per_cu(int G) {
    int n = 0;
    const hipError_t e = G == 1
        ? hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, lmhead_kernel<1, true, 1>, kThreads, 0)
        : hipOccupancyMaxActiveBlocksPerMultiprocessor(&n, lmhead_kernel<1, true, 3>, kThreads * 3, 0);
    return e == hipSuccess ? n : 0;
}

template <int G>
static hipError_t launch_lmhead_g(const LmheadParams &p, hipStream_t s, hipEvent_t after_rows) {
    const unsigned grid = (unsigned)(8 * (long long)p.RT * ((p.S + 7) / 8));
    const dim3 block(kThreads * G);
    const bool store = p.lg != nullptr;
    if (store)
        hipLaunchKernelGGL((lmhead_kernel<1, true, G>), dim3(grid), block, 0, s, p);
    else
        hipLaunchKernelGGL((lmhead_kernel<1, false, G>), dim3(grid), block, 0, s, p);
    hipError_t e = hipGetLastError();
    if (e != hipSuccess)
        return e;
    if (store && after_rows) {
        e = hipEventRecord(after_rows, s);
        if (e != hipSuccess)
            return e;
    }
    hipLaunchKernelGGL(lmhead_combine_kernel, dim3((unsigned)p.R), dim3(kThreads), 0, s, p);
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    if (store) {
        hipLaunchKernelGGL(lmhead_jsd_kernel, dim3((unsigned)(p.R * p.jc)), dim3(kThreads), 0, s, p);
    } else {
        // the recomputing pass on 64-row workgroups (its JSD epilogue is
        // VALU work that three workgroups per CU overlap with their loads
        // better than one 192-row workgroup does); its partials are per
        // (row, range), as the ranges are
        LmheadParams p1 = p;
        p1.G = 1;
        p1.RT = (int)((p.R + kLmRows - 1) / kLmRows);
        const unsigned grid1 = (unsigned)(8 * (long long)p1.RT * ((p.S + 7) / 8));
        hipLaunchKernelGGL((lmhead_kernel<2, false, 1>), dim3(grid1), dim3(kThreads), 0, s, p1);
        if ((e = hipGetLastError()) != hipSuccess)
            return e;
        if (after_rows) {
            e = hipEventRecord(after_rows, s);
            if (e != hipSuccess)
                return e;
        }
    }
    if ((e = hipGetLastError()) != hipSuccess)
        return e;
    hipLaunchKernelGGL(lmhead_finalize_kernel, dim3((unsigned)p.B), dim3(fin_threads(p.K + 1)), 0, s, p);
    return hipGetLastError();
}

hipError_t launch_lmhead(const LmheadParams &p, hipStream_t s, hipEvent_t after_rows) {
    return p.G == 3 ? launch_lmhead_g<3>(p, s, after_rows) : launch_lmhead_g<1>(p, s, after_rows);
}

} // namespace vwl
