// Device-side building blocks shared by the AsymSpec and RAPID kernels:
// element widening, wavefront/workgroup reductions, and the team protocol
// that lets the W workgroups of one logit row exchange per-chunk partials.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "vwl_internal.hpp"

namespace vwl {

constexpr int kWaves = kThreads / 64;
constexpr float kLog2e = 1.4426950408889634f;
constexpr double kLn2d = 0.6931471805599453;

enum { DT_F32 = 0, DT_BF16 = 1 };

// Elements per 16-byte vector and bytes per element of each dtype.
template <int DT> struct Elem;
template <> struct Elem<DT_F32> {
    static constexpr int kPerVec = 4;
    static constexpr int kBytes = 4;
};
template <> struct Elem<DT_BF16> {
    static constexpr int kPerVec = 8;
    static constexpr int kBytes = 2;
};

// Widen element j of a 16-byte vector to fp32 (exact for both dtypes).
template <int DT>
__device__ __forceinline__ float widen(const uint4 &v, int j);

template <>
__device__ __forceinline__ float widen<DT_F32>(const uint4 &v, int j) {
    const uint32_t w = j == 0 ? v.x : j == 1 ? v.y : j == 2 ? v.z : v.w;
    return __uint_as_float(w);
}

template <>
__device__ __forceinline__ float widen<DT_BF16>(const uint4 &v, int j) {
    const int k = j >> 1;
    const uint32_t w = k == 0 ? v.x : k == 1 ? v.y : k == 2 ? v.z : v.w;
    return (j & 1) ? __uint_as_float(w & 0xffff0000u) : __uint_as_float(w << 16);
}

// Record words: two floats in one 64-bit word, doubles as bit patterns.
__device__ __forceinline__ uint64_t pack2(float lo, float hi) {
    return (uint64_t)__float_as_uint(lo) | ((uint64_t)__float_as_uint(hi) << 32);
}
__device__ __forceinline__ float unpack_lo(uint64_t w) { return __uint_as_float((uint32_t)w); }
__device__ __forceinline__ float unpack_hi(uint64_t w) { return __uint_as_float((uint32_t)(w >> 32)); }
__device__ __forceinline__ double as_f64(uint64_t w) { return __longlong_as_double((long long)w); }
__device__ __forceinline__ uint64_t f64_bits(double x) { return (uint64_t)__double_as_longlong(x); }

// 2^k * x for an integer-valued float k <= 0.  Softmax references are kept
// as integers, so every change of reference is this exact power-of-two
// rescale (k below -1100 gives 0 for any finite sum).
__device__ __forceinline__ double scale_pow2(double x, float k) {
    return ldexp(x, (int)fmaxf(k, -1100.0f));
}

// One element of a row, widened to fp32.
template <int DT>
__device__ __forceinline__ float load_scalar(const void *base, size_t idx) {
    if (DT == DT_BF16) {
        const uint16_t h = static_cast<const uint16_t *>(base)[idx];
        return __uint_as_float(static_cast<uint32_t>(h) << 16);
    }
    return static_cast<const float *>(base)[idx];
}

// ---------------------------------------------------------------------------
// Wavefront all-reductions (64 lanes) without LDS: two DPP steps within each
// quad (lane ^ 1, lane ^ 2), the half-row and row mirrors (combining groups of
// 4 and 8), then the gfx950 lane swaps across 16-lane rows and 32-lane
// halves.  Every step combines two partial results with a commutative
// operation, so all lanes end with the same bits, in a fixed order: the
// results are deterministic.
// ---------------------------------------------------------------------------
// Every lane has a valid source lane under the in-row controls used here, so
// the move needs no "old" value and the compiler may fold it into its user.
template <int CTRL>
__device__ __forceinline__ int dpp_i(int x) {
    return __builtin_amdgcn_mov_dpp(x, CTRL, 0xf, 0xf, false);
}
constexpr int kDppXor1 = 0xB1;       // quad_perm [1,0,3,2]
constexpr int kDppXor2 = 0x4E;       // quad_perm [2,3,0,1]
constexpr int kDppHalfMirror = 0x141;
constexpr int kDppMirror = 0x140;
constexpr int kDppBcast15 = 0x142;   // lane 15 of each row to the next row
constexpr int kDppBcast31 = 0x143;   // lane 31 to rows 2 and 3
// A row broadcast written to the rows in ROWS only; the other rows get `old`.
template <int CTRL, int ROWS>
__device__ __forceinline__ int dpp_bcast(int old, int x) {
    return __builtin_amdgcn_update_dpp(old, x, CTRL, ROWS, 0xf, false);
}

// One combining step with the DPP operand folded into the max / min: x gets
// op(x, x from the lane CTRL selects); rows outside ROWS keep x.  Written as
// instructions so that no NaN canonicalisation of the moved value is added.
// Wait states: the first step of a chain allows for any earlier VALU write
// (five: a write of EXEC), the later ones for the previous step's write of x
// (two), and each chain ends with two more before the next reader of x.
#define VWL_DPP_STEP(NOPS, OP, CTRL_TEXT, ROWS_TEXT)                                            \
    asm("s_nop " NOPS "\n\t" OP " %0, %0, %0 " CTRL_TEXT " row_mask:" ROWS_TEXT " bank_mask:0xf" \
        : "+v"(x))
#define VWL_DPP_END() asm("s_nop 1" : "+v"(x))
__device__ __forceinline__ float fmax_dpp_steps(float x) { // in-row steps
    VWL_DPP_STEP("4", "v_max_f32_dpp", "quad_perm:[1,0,3,2]", "0xf");
    VWL_DPP_STEP("1", "v_max_f32_dpp", "quad_perm:[2,3,0,1]", "0xf");
    VWL_DPP_STEP("1", "v_max_f32_dpp", "row_half_mirror", "0xf");
    VWL_DPP_STEP("1", "v_max_f32_dpp", "row_mirror", "0xf");
    return x;
}
__device__ __forceinline__ int imin_dpp_steps(int x) {
    VWL_DPP_STEP("4", "v_min_i32_dpp", "quad_perm:[1,0,3,2]", "0xf");
    VWL_DPP_STEP("1", "v_min_i32_dpp", "quad_perm:[2,3,0,1]", "0xf");
    VWL_DPP_STEP("1", "v_min_i32_dpp", "row_half_mirror", "0xf");
    VWL_DPP_STEP("1", "v_min_i32_dpp", "row_mirror", "0xf");
    return x;
}
// Plain maximum of two floats without input canonicalisation.
__device__ __forceinline__ float fmax_raw(float a, float b) {
    float r;
    asm("v_max_f32 %0, %1, %2" : "=v"(r) : "v"(a), "v"(b));
    return r;
}

// Partner values across 16-lane rows and across 32-lane halves: returns the
// pair (own, partner) in some order; only commutative uses are made of it.
__device__ __forceinline__ void swap16(int x, int &u, int &v) {
    const auto p = __builtin_amdgcn_permlane16_swap(x, x, false, false);
    u = p[0];
    v = p[1];
}
__device__ __forceinline__ void swap32(int x, int &u, int &v) {
    const auto p = __builtin_amdgcn_permlane32_swap(x, x, false, false);
    u = p[0];
    v = p[1];
}

__device__ __forceinline__ float wave_max(float x) {
    x = fmax_dpp_steps(x);
    VWL_DPP_END();
    int u, v;
    swap16(__float_as_int(x), u, v);
    x = fmax_raw(__int_as_float(u), __int_as_float(v));
    swap32(__float_as_int(x), u, v);
    return fmax_raw(__int_as_float(u), __int_as_float(v));
}

__device__ __forceinline__ int wave_min_int(int x) {
    x = imin_dpp_steps(x);
    VWL_DPP_END();
    int u, v;
    swap16(x, u, v);
    x = min(u, v);
    swap32(x, u, v);
    return min(u, v);
}

template <int CTRL>
__device__ __forceinline__ double dpp_d(double x) {
    const long long b = __double_as_longlong(x);
    const int lo = dpp_i<CTRL>((int)b), hi = dpp_i<CTRL>((int)(b >> 32));
    return __longlong_as_double(((long long)hi << 32) | (long long)(uint32_t)lo);
}

__device__ __forceinline__ double wave_sum(double x) {
    x += dpp_d<kDppXor1>(x);
    x += dpp_d<kDppXor2>(x);
    x += dpp_d<kDppHalfMirror>(x);
    x += dpp_d<kDppMirror>(x);
    {
        const long long b = __double_as_longlong(x);
        int l0, l1, h0, h1;
        swap16((int)b, l0, l1);
        swap16((int)(b >> 32), h0, h1);
        x = __longlong_as_double(((long long)h0 << 32) | (long long)(uint32_t)l0) +
            __longlong_as_double(((long long)h1 << 32) | (long long)(uint32_t)l1);
    }
    {
        const long long b = __double_as_longlong(x);
        int l0, l1, h0, h1;
        swap32((int)b, l0, l1);
        swap32((int)(b >> 32), h0, h1);
        x = __longlong_as_double(((long long)h0 << 32) | (long long)(uint32_t)l0) +
            __longlong_as_double(((long long)h1 << 32) | (long long)(uint32_t)l1);
    }
    return x;
}

// Reductions whose result is needed in lane 63 only (the wave's entry of a
// workgroup reduction): after the in-row steps every lane of a row holds
// its row's result; row 1 then adds row 0 and row 3 adds row 2 (broadcast of
// lane 15), and rows 2 and 3 add lane 31 (rows 0 and 1).  The order is fixed,
// so the result is deterministic.  Other lanes end with partial results.
__device__ __forceinline__ float wave_max_last(float x) {
    x = fmax_dpp_steps(x);
    VWL_DPP_STEP("1", "v_max_f32_dpp", "row_bcast:15", "0xa");
    VWL_DPP_STEP("1", "v_max_f32_dpp", "row_bcast:31", "0xc");
    VWL_DPP_END();
    return x;
}

__device__ __forceinline__ int wave_min_last(int x) {
    x = imin_dpp_steps(x);
    VWL_DPP_STEP("1", "v_min_i32_dpp", "row_bcast:15", "0xa");
    VWL_DPP_STEP("1", "v_min_i32_dpp", "row_bcast:31", "0xc");
    VWL_DPP_END();
    return x;
}

template <int CTRL, int ROWS>
__device__ __forceinline__ double dpp_d_bcast(double x) { // rows outside ROWS get +0.0
    const long long b = __double_as_longlong(x);
    const int lo = dpp_bcast<CTRL, ROWS>(0, (int)b), hi = dpp_bcast<CTRL, ROWS>(0, (int)(b >> 32));
    return __longlong_as_double(((long long)hi << 32) | (long long)(uint32_t)lo);
}

__device__ __forceinline__ double wave_sum_last(double x) {
    x += dpp_d<kDppXor1>(x);
    x += dpp_d<kDppXor2>(x);
    x += dpp_d<kDppHalfMirror>(x);
    x += dpp_d<kDppMirror>(x);
    x += dpp_d_bcast<kDppBcast15, 0xa>(x);
    x += dpp_d_bcast<kDppBcast31, 0xc>(x);
    return x;
}

// N independent lane-63 reductions advanced together, one step across all N
// values at a time, so that their dependency chains overlap.
#define VWL_DPPN_I(OP, CTRL, ROWS, K) OP " %" #K ", %" #K ", %" #K " " CTRL " row_mask:" ROWS " bank_mask:0xf\n\t"
#define VWL_DPPN_STEP(NOPS, OP, CTRL, ROWS)                                                              \
    do {                                                                                                 \
        if constexpr (N == 1)                                                                            \
            asm("s_nop " NOPS "\n\t" VWL_DPPN_I(OP, CTRL, ROWS, 0) : "+v"(x[0]));                        \
        else if constexpr (N == 2)                                                                       \
            asm("s_nop " NOPS "\n\t" VWL_DPPN_I(OP, CTRL, ROWS, 0) VWL_DPPN_I(OP, CTRL, ROWS, 1)         \
                : "+v"(x[0]), "+v"(x[1]));                                                               \
        else if constexpr (N == 3)                                                                       \
            asm("s_nop " NOPS "\n\t" VWL_DPPN_I(OP, CTRL, ROWS, 0) VWL_DPPN_I(OP, CTRL, ROWS, 1)         \
                    VWL_DPPN_I(OP, CTRL, ROWS, 2)                                                        \
                : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]));                                                   \
        else                                                                                             \
            asm("s_nop " NOPS "\n\t" VWL_DPPN_I(OP, CTRL, ROWS, 0) VWL_DPPN_I(OP, CTRL, ROWS, 1)         \
                    VWL_DPPN_I(OP, CTRL, ROWS, 2) VWL_DPPN_I(OP, CTRL, ROWS, 3)                          \
                : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));                                       \
    } while (0)

#define VWL_DPPN_END()                                                                                   \
    do {                                                                                                 \
        if constexpr (N == 1)                                                                            \
            asm("s_nop 1" : "+v"(x[0]));                                                                 \
        else if constexpr (N == 2)                                                                       \
            asm("s_nop 1" : "+v"(x[0]), "+v"(x[1]));                                                     \
        else if constexpr (N == 3)                                                                       \
            asm("s_nop 1" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]));                                         \
        else                                                                                             \
            asm("s_nop 1" : "+v"(x[0]), "+v"(x[1]), "+v"(x[2]), "+v"(x[3]));                             \
    } while (0)

template <int N>
__device__ __forceinline__ void wave_max_last_n(float (&x)[N]) {
    static_assert(N >= 1 && N <= 4, "up to four values");
    VWL_DPPN_STEP("4", "v_max_f32_dpp", "quad_perm:[1,0,3,2]", "0xf");
    VWL_DPPN_STEP("1", "v_max_f32_dpp", "quad_perm:[2,3,0,1]", "0xf");
    VWL_DPPN_STEP("1", "v_max_f32_dpp", "row_half_mirror", "0xf");
    VWL_DPPN_STEP("1", "v_max_f32_dpp", "row_mirror", "0xf");
    VWL_DPPN_STEP("1", "v_max_f32_dpp", "row_bcast:15", "0xa");
    VWL_DPPN_STEP("1", "v_max_f32_dpp", "row_bcast:31", "0xc");
    VWL_DPPN_END();
}

template <int N>
__device__ __forceinline__ void wave_sum_last_n(double (&x)[N]) {
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] += dpp_d<kDppXor1>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] += dpp_d<kDppXor2>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] += dpp_d<kDppHalfMirror>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] += dpp_d<kDppMirror>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] += dpp_d_bcast<kDppBcast15, 0xa>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] += dpp_d_bcast<kDppBcast31, 0xc>(x[i]);
}

// Workgroup sums whose result one lane needs (lane 63 of wave 0): two quad
// steps in every wave, the 64 quad partials of each value through LDS, then
// wave 0 alone folds them.  Every wave writes its partials before the
// barrier the caller places next; `finish` (wave 0, after that barrier)
// returns the sums in lane 63, in one fixed order.  `lds` holds 64*N doubles.
template <int N>
__device__ __forceinline__ void quad_sum_post(double (&x)[N], double *lds) {
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] += dpp_d<kDppXor1>(x[i]);
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] += dpp_d<kDppXor2>(x[i]);
    if ((threadIdx.x & 3) == 0) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            lds[i * 64 + (threadIdx.x >> 2)] = x[i];
    }
}
template <int N>
__device__ __forceinline__ void quad_sum_finish(double (&x)[N], const double *lds) {
    const int lane = threadIdx.x & 63;
#pragma unroll
    for (int i = 0; i < N; ++i)
        x[i] = lds[i * 64 + lane];
    wave_sum_last_n<N>(x);
}

// Workgroup barrier for LDS data only: the wave's LDS operations complete,
// then s_barrier.  Unlike __syncthreads() it does not wait for the wave's
// global loads, so staging loads in flight (direct global -> LDS loads of a
// later row) stay in flight across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory"); }

template <bool LDS_ONLY>
__device__ __forceinline__ void wg_barrier() {
    if constexpr (LDS_ONLY)
        lds_barrier();
    else
        __syncthreads();
}

// Workgroup reductions: wave results go through LDS and every thread combines
// the WAVES values in the same order, so all threads hold the same result.
// With TRAIL = false the closing barrier is left out: the caller guarantees
// that another workgroup barrier separates the reads of `lds` from its next
// write.  WAVES is the workgroup's wave count (kWaves unless stated).  With
// LDS_ONLY the barriers are LDS-only (lds_barrier), for callers with staging
// loads in flight.
template <int N, bool TRAIL = true, int WAVES = kWaves, bool LDS_ONLY = false>
__device__ __forceinline__ void block_max(float (&x)[N], float *lds /* WAVES*N */) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    float m[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        m[i] = x[i];
    wave_max_last_n<N>(m);
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            lds[wave * N + i] = m[i];
    }
    wg_barrier<LDS_ONLY>();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        float r = lds[i];
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
            r = fmax_raw(r, lds[w * N + i]);
        x[i] = r;
    }
    if (TRAIL)
        wg_barrier<LDS_ONLY>();
}

template <int N, bool TRAIL = true, int WAVES = kWaves, bool LDS_ONLY = false>
__device__ __forceinline__ void block_sum(double (&x)[N], double *lds /* WAVES*N */) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double m[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        m[i] = x[i];
    wave_sum_last_n<N>(m);
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            lds[wave * N + i] = m[i];
    }
    wg_barrier<LDS_ONLY>();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        double r = lds[i];
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
            r += lds[w * N + i];
        x[i] = r;
    }
    if (TRAIL)
        wg_barrier<LDS_ONLY>();
}

// Sums of N doubles and the minimum of one int in a single LDS round.
template <int N, bool TRAIL = true, int WAVES = kWaves>
__device__ __forceinline__ void block_sum_min(double (&x)[N], int &imin, double *lds /* WAVES*N */,
                                              int *ldsi /* WAVES */) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    double m[N];
#pragma unroll
    for (int i = 0; i < N; ++i)
        m[i] = x[i];
    wave_sum_last_n<N>(m);
    const int mi = wave_min_last(imin);
    if (lane == 63) {
#pragma unroll
        for (int i = 0; i < N; ++i)
            lds[wave * N + i] = m[i];
        ldsi[wave] = mi;
    }
    __syncthreads();
#pragma unroll
    for (int i = 0; i < N; ++i) {
        double r = lds[i];
#pragma unroll
        for (int w = 1; w < WAVES; ++w)
            r += lds[w * N + i];
        x[i] = r;
    }
    int r = ldsi[0];
#pragma unroll
    for (int w = 1; w < WAVES; ++w)
        r = min(r, ldsi[w]);
    imin = r;
    if (TRAIL)
        __syncthreads();
}

template <bool LDS_ONLY = false>
__device__ __forceinline__ int block_min_int(int x, int *lds /* kWaves */) {
    const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6;
    const int m = wave_min_last(x);
    if (lane == 63)
        lds[wave] = m;
    wg_barrier<LDS_ONLY>();
    int r = lds[0];
#pragma unroll
    for (int w = 1; w < kWaves; ++w)
        r = min(r, lds[w]);
    wg_barrier<LDS_ONLY>();
    return r;
}

// ---------------------------------------------------------------------------
// Data exchanged between workgroups of one launch.
//
// Every such word (records, counters, per-row results) is written and read
// only through device-scope (agent) atomic loads and stores, which are
// coherent across the XCDs by themselves.  The one ordering the protocol
// needs -- a record's stores are complete before the counter increment that
// announces it -- is a wait for the issuing thread's outstanding memory
// operations.  This avoids acquire/release fences, which on this target
// write back and invalidate the whole L2 on every call (and on every poll of
// a wait loop).
// ---------------------------------------------------------------------------
__device__ __forceinline__ void wait_stores_complete() {
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory");
}
__device__ __forceinline__ uint32_t ld_counter(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
// Publish: all earlier stores of this thread complete, then the increment.
__device__ __forceinline__ uint32_t publish_add(uint32_t *p, uint32_t v) {
    wait_stores_complete();
    const uint32_t old = __hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    __asm__ volatile("s_waitcnt vmcnt(0)" ::: "memory"); // later loads issue after the result
    return old;
}
// Publish without waiting for the counter's result.
__device__ __forceinline__ void publish_add_nr(uint32_t *p, uint32_t v) {
    wait_stores_complete();
    (void)__hip_atomic_fetch_add(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint32_t *p, uint32_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_relaxed(uint64_t *p, uint64_t v) {
    __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint32_t ld_relaxed(const uint32_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ uint64_t ld_relaxed(const uint64_t *p) {
    return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}
__device__ __forceinline__ void st_f64(double *p, double v) {
    st_relaxed(reinterpret_cast<uint64_t *>(p), static_cast<uint64_t>(__double_as_longlong(v)));
}
__device__ __forceinline__ double ld_f64(const double *p) {
    return __longlong_as_double(static_cast<long long>(ld_relaxed(reinterpret_cast<const uint64_t *>(p))));
}

// Wall clock (constant 100 MHz) used to bound every wait.
constexpr uint64_t kWaitLimitTicks = 200000000ull; // ~2 s

// Wait until *ctr >= target.  Called by one thread.  Returns false when the
// bound expired (the caller records a timeout and abandons its remaining work).
__device__ __forceinline__ bool wait_at_least(const uint32_t *ctr, uint32_t target) {
    if (ld_counter(ctr) >= target)
        return true;
    const uint64_t t0 = wall_clock64();
    while (ld_counter(ctr) < target) {
        __builtin_amdgcn_s_sleep(1);
        if (wall_clock64() - t0 > kWaitLimitTicks)
            return false;
    }
    __asm__ volatile("" ::: "memory");
    return true;
}

// As wait_at_least, telling also whether any waiting was needed:
// 2 = the target was already reached at the first look, 1 = reached after
// waiting, 0 = the bound expired.
__device__ __forceinline__ uint32_t wait_at_least_seen(const uint32_t *ctr, uint32_t target) {
    if (ld_counter(ctr) >= target)
        return 2u;
    return wait_at_least(ctr, target) ? 1u : 0u;
}

__device__ __forceinline__ void set_dev_err(int32_t *dev_err, int bits) {
    if (dev_err)
        __hip_atomic_fetch_or(dev_err, bits, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// ---------------------------------------------------------------------------
// Geometry of one row split over W members.
//
// A row of V elements starting at element offset `row_off` of a 16-byte
// aligned tensor has `head` leading elements before its first 16-byte
// boundary, `nb` whole vectors, then `tail` trailing elements.  Member w
// takes the `chunk` vectors starting at w * chunk (the last member of a row
// may take fewer; `chunk` is fixed per launch, so no division is needed
// here); head and tail elements are handled one per lane by the first and
// the last member.
// ---------------------------------------------------------------------------
template <int DT>
struct RowSplit {
    long long vec0;   // first vector (index into the tensor viewed as uint4)
    int nv;           // vectors of this member
    int first_elem;   // element index within the row of this member's first vector
    int nsc;          // scalar elements of this member (<= 2*(kPerVec-1))
    int sc_idx0;      // row element index of scalar 0 (head)
    int n_head;       // how many of the scalars are head elements
    int sc_idx1;      // row element index of the first tail scalar
};

template <int DT>
__device__ __forceinline__ RowSplit<DT> row_split(long long row, int V, int W, int w, int chunk) {
    constexpr int EPV = Elem<DT>::kPerVec;
    const long long off = row * (long long)V;                 // element offset of the row
    int head = (int)((EPV - (int)(off & (EPV - 1))) & (EPV - 1));
    if (head > V)
        head = V;
    const int nb = (V - head) / EPV;
    const int tail = V - head - nb * EPV;
    const int v0 = min(w * chunk, nb), v1 = min(v0 + chunk, nb);
    RowSplit<DT> s;
    s.vec0 = (off + head) / EPV + v0;
    s.nv = v1 - v0;
    s.first_elem = head + v0 * EPV;
    s.n_head = (w == 0) ? head : 0;
    s.sc_idx0 = 0;
    s.sc_idx1 = head + nb * EPV;
    s.nsc = s.n_head + ((w == W - 1) ? tail : 0);
    return s;
}

template <int DT>
__device__ __forceinline__ int scalar_index(const RowSplit<DT> &s, int k) {
    return k < s.n_head ? s.sc_idx0 + k : s.sc_idx1 + (k - s.n_head);
}

} // namespace vwl
