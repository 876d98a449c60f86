// Device helpers shared by the gfx950 kernels: exact fixed-point
// requantisation, byte packing and the barrier / wait primitives the
// software pipelines use.
#pragma once

#include <hip/hip_runtime.h>

namespace ifx {

// s_waitcnt vmcnt(n), expcnt/lgkmcnt unconstrained (gfx9 encoding).  Vector
// loads complete in issue order, so "at most n outstanding" guarantees every
// load older than the last n loads has landed, whatever stores are pending.
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Workgroup barrier for LDS filled by DMA: every wave has already waited for
// its own loads, and LDS needs no cache maintenance, so a bare s_barrier
// publishes them (__syncthreads would add a fence that drains every load in
// flight).  The empty asm keeps the compiler from moving LDS accesses across.
__device__ __forceinline__ void ring_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Intra-wave LDS hand-over (lanes read what other lanes of the same wave
// wrote): LDS executes a wave's accesses in order; only compiler reordering
// has to be prevented.
__device__ __forceinline__ void wave_lds_sync()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
}

// Workgroup barrier after this wave's own LDS writes (ds_write): wait for
// them to complete, then a bare s_barrier (no fence, so vector memory
// operations in flight, loads and stores, stay in flight).
__device__ __forceinline__ void lds_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_waitcnt(0xc07f);  // lgkmcnt(0); vmcnt, expcnt unconstrained
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// Requantisation, exact for every |y| < 2^31, 0 <= m < 2^31, 0 <= sh <= 31:
//   q = round_half_away_from_zero(y * m / 2^(31+sh))
//     = floor((y*m + 2^(30+sh) - [y<0]) / 2^(31+sh))     (floor = arithmetic shift)
// General form: one 64-bit product and one 64-bit shift.
__device__ __forceinline__ int requant_any(int y, int m, int sh)
{
    long long p = (long long)y * (long long)m + (1ll << (30 + sh)) - (y < 0 ? 1 : 0);
    return (int)(p >> (31 + sh));
}

// sh >= 2: 2^(30+sh) - [y<0] has high word 2^(sh-2) + sgn and low word sgn
// (sgn = y >> 31), so the sum is one v_mad_i64_i32 and the quotient is the
// high word shifted by sh - 1.
__device__ __forceinline__ int requant_fast(int y, int m, int rnd_hi, int sh_m1)
{
    int sgn = y >> 31;
    long long add = (long long)(((unsigned long long)(unsigned)(rnd_hi + sgn) << 32) | (unsigned)sgn);
    long long p = (long long)y * (long long)m + add;
    return ((int)(p >> 32)) >> sh_m1;
}

// sh >= 2 followed by a ReLU with no shortcut: for y < 0 the result is <= 0
// either way and the ReLU clears it, so the [y<0] tie correction is dropped.
__device__ __forceinline__ int requant_relu(int y, int m, int rnd_hi, int sh_m1)
{
    long long add = (long long)((unsigned long long)(unsigned)rnd_hi << 32);
    long long p = (long long)y * (long long)m + add;
    return ((int)(p >> 32)) >> sh_m1;
}

// Pack the low bytes of four int32 values (already in [-128, 127]).
__device__ __forceinline__ unsigned pack4(int q0, int q1, int q2, int q3)
{
    unsigned lo = __builtin_amdgcn_perm((unsigned)q1, (unsigned)q0, 0x0c0c0400u);
    unsigned hi = __builtin_amdgcn_perm((unsigned)q3, (unsigned)q2, 0x0c0c0400u);
    return __builtin_amdgcn_perm(hi, lo, 0x05040100u);
}

}  // namespace ifx
