// Staging of a row's chunk from HBM into LDS with direct global -> LDS
// loads, shared by the row kernels: the [tensor][vector slot][thread]
// layout, the per-wave issue of one tensor's vectors from a uniform base,
// the head/tail scalars of a row, and the LDS-only barrier.
#pragma once

#include "vwl_device.hpp"
#include "vwl_internal.hpp"

namespace vwl {

// LDS staging of one row's chunk: [tensor][vector slot][thread], 16 bytes
// each.  Every lane later reads back exactly the vectors it issued itself,
// so only its own wave's loads have to be complete.
template <int NV, int NT>
struct AsymStage {
    uint4 v[NT][NV][kThreads];
};

// Direct global -> LDS load of one 16-byte vector per lane from the lane's
// own address (the LDS address of the wave is uniform; lane L lands at
// lds_wave_base + 16*L).  The compiler tracks these loads: it waits for them
// before any LDS access that may alias them.
__device__ __forceinline__ void g2lds16(const uint4 *src, uint4 *lds_wave_base) {
    __builtin_amdgcn_global_load_lds(static_cast<const void *>(src),
                                     (__attribute__((address_space(3))) void *)(lds_wave_base), 16, 0, 0);
}

// Direct global -> LDS load of one 16-byte vector per lane: the wave reads
// the 64 vectors at the uniform `sbase` (lane L at sbase + 16*L) into LDS
// at the uniform `lds_wave` (lane L at lds_wave + 16*L).  Issued from
// inline assembly, so the compiler does not treat later LDS accesses as
// possibly aliasing it and adds no wait for it before them; the kernel
// waits for these loads itself (vmcnt(0) and a barrier before the staged
// row is read).  The address is an SGPR base plus the lane's byte offset,
// with no vector arithmetic.  The compiler does not check hazards against
// the instructions inside the assembly, so it begins with the wait states
// the hardware requires before a vector memory instruction reads an SGPR
// that a VALU instruction (here v_readfirstlane) may have just written (5),
// which also covers the one after a write of M0.
__device__ __forceinline__ const uint4 *uniform_ptr(const uint4 *p) {
    const uint64_t a = reinterpret_cast<uint64_t>(p);
    const uint32_t lo = __builtin_amdgcn_readfirstlane((uint32_t)a);
    const uint32_t hi = __builtin_amdgcn_readfirstlane((uint32_t)(a >> 32));
    return reinterpret_cast<const uint4 *>(((uint64_t)hi << 32) | lo);
}
__device__ __forceinline__ void g2lds16_wave(const uint4 *sbase, const uint4 *lds_wave) {
    const uint4 *ub = uniform_ptr(sbase);
    const uint32_t m0 = __builtin_amdgcn_readfirstlane((uint32_t)reinterpret_cast<uintptr_t>(lds_wave));
    const uint32_t voff = (threadIdx.x & 63) * 16u;
    asm volatile("s_nop 4\n\tglobal_load_lds_dwordx4 %0, %1" ::"v"(voff), "s"(ub), "{m0}"(m0) : "memory");
}


// Stream row r's chunk into LDS (waves 1-3: wave x+1 issues all of tensor x;
// wave 1 idles when a is not read, wave 3 when t is not).
template <int DT, int NV, int NT, bool READ_A>
__device__ __forceinline__ void prefetch_bulk(AsymStage<NV, NT> &stage, long long r, int V, int W, int member,
                                              int chunk, const uint4 *A4, const uint4 *B4, const uint4 *T4) {
    const int lane = threadIdx.x & 63;
    const RowSplit<DT> s = row_split<DT>(r, V, W, member, chunk);
    const int x = __builtin_amdgcn_readfirstlane((int)(threadIdx.x >> 6)) - 1;
    if ((!READ_A && x == 0) || x >= NT)
        return;
    const uint4 *base = T4;
    if (x == 0)
        base = A4;
    else if (x == 1)
        base = B4;
    const uint4 *ub = uniform_ptr(base + s.vec0); // the per-load bases below are scalar adds
    uint4 *dst = &stage.v[x][0][0];
    if (s.nv >= NV * kThreads) { // the whole slot (uniform)
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int v = 0; v < kWaves; ++v)
                g2lds16_wave(ub + j * kThreads + v * 64, dst + j * kThreads + v * 64);
    } else {
        const int rem = s.nv - lane; // this lane loads the sub-blocks that start below rem
#pragma unroll
        for (int j = 0; j < NV; ++j)
#pragma unroll
            for (int v = 0; v < kWaves; ++v) {
                if (j * kThreads + v * 64 < rem)
                    g2lds16_wave(ub + j * kThreads + v * 64, dst + j * kThreads + v * 64);
            }
    }
}

// Head/tail scalars of row r (wave 0's first lanes), as raw bits: they are
// widened when the row is taken, so the loads stay in flight until then.
// Every lane of wave 0 loads (lanes past the scalars read a valid element of
// the row and ignore it), so no merge of the loaded registers forces an early
// wait either.
template <int DT>
__device__ __forceinline__ uint32_t load_raw(const void *base, size_t idx) {
    if (DT == DT_BF16)
        return static_cast<uint32_t>(static_cast<const uint16_t *>(base)[idx]);
    return static_cast<const uint32_t *>(base)[idx];
}
template <int DT>
__device__ __forceinline__ float widen_raw(uint32_t x) {
    return DT == DT_BF16 ? __uint_as_float(x << 16) : __uint_as_float(x);
}

template <int DT, bool READ_A, bool READ_T>
__device__ __forceinline__ void prefetch_scalars(long long r, int V, int W, int member, int chunk, const void *a,
                                                 const void *b, const void *t, uint32_t &na, uint32_t &nb,
                                                 uint32_t &nt) {
    const RowSplit<DT> s = row_split<DT>(r, V, W, member, chunk);
    const int k = (int)threadIdx.x < s.nsc ? (int)threadIdx.x : 0;
    const size_t off = (size_t)r * (size_t)V + (s.nsc > 0 ? (size_t)scalar_index<DT>(s, k) : 0);
    if (READ_A)
        na = load_raw<DT>(a, off);
    nb = load_raw<DT>(b, off);
    if (READ_T)
        nt = load_raw<DT>(t, off);
}

} // namespace vwl
