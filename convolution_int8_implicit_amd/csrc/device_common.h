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

// Requantisation, exact for every int32 y (-2^31 <= y < 2^31), 0 <= m < 2^31, 0 <= sh <= 31:
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

// ---------------------------------------------------------------------------
// Buffer-resource loads and the shared tile epilogue of the convolution kernels
// ---------------------------------------------------------------------------
typedef int ifx_v4i __attribute__((ext_vector_type(4)));

// Direct buffer -> LDS load: each lane's `size` bytes land at lds + lane * size.
__device__ void ifx_raw_buffer_load_lds(ifx_v4i rsrc, __attribute__((address_space(3))) void *lds, int size,
                                        unsigned voffset, int soffset, int offset,
                                        int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

// Buffer store of 16 bytes; a lane whose offset lies past the resource's range writes nothing.
__device__ void ifx_raw_buffer_store_v4i32(ifx_v4i vdata, ifx_v4i rsrc, unsigned voffset, int soffset,
                                           int aux) __asm("llvm.amdgcn.raw.buffer.store.v4i32");

namespace ifx {

typedef ifx_v4i v4i;

constexpr int kLdsBytes = 160 * 1024;  // LDS per CU on gfx950
// The second operand of __launch_bounds__ on this target is the minimum number of waves per SIMD
// (which caps the registers per wave at 512 / that), not workgroups per CU: workgroups of
// `threads` threads, `per_cu` of them resident on a CU's four SIMDs.
constexpr int waves_per_simd(int threads, int per_cu) { return (threads / 64 * per_cu + 3) / 4; }

constexpr unsigned kOOB = 0x80000000u;  // offset past every buffer range: loads return zero
constexpr int kCachePolicyNT = 2;       // buffer instruction cache-policy operand: non-temporal

// Buffer resource (gfx9 layout): 48-bit base, stride 0, byte range, raw-buffer config word.
__device__ __forceinline__ v4i make_rsrc(const void *base, long long range)
{
    unsigned long long a = (unsigned long long)base;
    unsigned r = (unsigned)(range < 0 ? 0 : (range > 0x7ffffff0ll ? 0x7ffffff0ll : range));
    v4i v;
    v.x = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
    v.y = __builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32) & 0xffff);
    v.z = __builtin_amdgcn_readfirstlane((int)r);
    v.w = 0x00020000;
    return v;
}

__device__ __forceinline__ void load16_lds(v4i rsrc, int8_t *lds_wave_base, unsigned voff)
{
    ifx_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)(lds_wave_base), 16, voff, 0, 0, 0);
}

// The same for data read once (streamed): the non-temporal policy keeps it from
// displacing reused operands in L2 and the MALL.
__device__ __forceinline__ void load16_lds_stream(v4i rsrc, int8_t *lds_wave_base, unsigned voff)
{
    ifx_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)(lds_wave_base), 16, voff, 0, 0,
                            kCachePolicyNT);
}

// 16-byte store of output written once, non-temporal.
__device__ __forceinline__ void store16_stream(int8_t *p, v4i v) { __builtin_nontemporal_store(v, (v4i *)p); }

// floor(n / d) for 0 <= n < 2^31 with the host-computed magic of d (mul == 0 means d == 1).
__device__ __forceinline__ int fdiv(int n, unsigned mul, int shr)
{
    return mul == 0 ? n : (int)(__umulhi((unsigned)n, mul) >> shr);
}

// 16-byte-chunk XOR swizzle of a 64-byte LDS row (chunk k of row r stored at slot k ^ swz(r)).
// A ds_read_b128 serves lanes {0-7, 24-31}, {8-15, 16-23}, {32-39, 56-63}, {40-47, 48-55}
// one group per cycle; a lane (c = l % 16, g = l / 16) reads chunk g of row 16 t + c (weights)
// or 16 t + 4(c % 4) + c / 4 (pixels).  With swz = (r / 4 ^ r) % 4 every group of either
// pattern reaches 16 distinct 16-byte bank slots.
__device__ __forceinline__ int swz(int row) { return ((row >> 2) ^ row) & 3; }

// Compile-time tags for dispatching a wave-uniform runtime mode into template code.
struct Slot0 {
    static constexpr int value = 0;
};
struct Slot1 {
    static constexpr int value = 1;
};
struct Slot2 {
    static constexpr int value = 2;
};

// Requantisation parameters of the four output channels a lane owns.
struct RqLane {
    int bias[4];       // added to the accumulator (modes 0 and 2; 0 when it already holds the bias)
    int mul[4], shf[4];
    int rnd[4], shm[4];  // 2^(shift-2) and shift-1 (modes 1 and 2)
    long long add[4];  // mode 1: bias*mult + 2^(30+shift), the whole rounding addend
};

// Set up the lane's channels ocl .. ocl+3 (channels >= oc: mult 0, so they give 0) and pick the
// wave's mode:
//   0  any shift: one general requant_any per element;
//   1  every shift >= 2 and no rounding tie possible (or ReLU without a shortcut, where a tie
//      on a negative value ends at 0 either way): q = hi(acc*m + add) >> (shift-1), one
//      v_mad_i64_i32 and one shift per element, the bias folded into `add`;
//   2  every shift >= 2: requant_fast, which carries the [y<0] tie correction.
// A tie (y*m/2^(31+s) exactly halfway) needs v2(y) + v2(m) = 30 + s.  An int32 y has
// v2(y) <= 31, with 31 only for y = -2^31 (a bias of INT32_MIN on a zero sum reaches it), so no
// tie can happen when m has at most s - 2 trailing zero bits (or m == 0).
template <bool RES, bool RELU>
__device__ __forceinline__ int rq_setup(RqLane &r, v4i bias4, v4i mult4, v4i shift4, bool bias_in_acc, int ocl,
                                        int oc)
{
    bool fast = true, tiefree = true;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
        const bool v = ocl + tn < oc;
        const int b = v && !bias_in_acc ? bias4[tn] : 0;
        const int m = v ? mult4[tn] : 0;
        const int s = v ? shift4[tn] : 2;
        r.bias[tn] = b;
        r.mul[tn] = m;
        r.shf[tn] = s;
        r.rnd[tn] = 1 << ((s - 2) & 31);
        r.shm[tn] = s - 1;
        r.add[tn] = (long long)b * (long long)m + (long long)((unsigned long long)(unsigned)r.rnd[tn] << 32);
        fast = fast && s >= 2;
        tiefree = tiefree && (m == 0 || (int)__builtin_ctz((unsigned)m) + 1 < s);
    }
    if (!__all(fast)) return 0;
    if ((!RES && RELU) || __all(tiefree)) return 1;
    return 2;
}

// One tile row of a lane: its 4 channels of row 16tm + 4i + g requantised (mode MODE), plus the
// shortcut bytes rr when RES, clamped (ReLU or not) and packed into one word.
template <int MODE, bool RES, bool RELU, int TM>
__device__ __forceinline__ unsigned requant_row(const v4i (&acc)[TM][4], int tm, int i, const RqLane &r, unsigned rr)
{
    int q[4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
        int v;
        if (MODE == 0) {
            v = requant_any(acc[tm][tn][i] + r.bias[tn], r.mul[tn], r.shf[tn]);
        } else if (MODE == 1) {
            const long long p = (long long)acc[tm][tn][i] * (long long)r.mul[tn] + r.add[tn];
            v = ((int)(p >> 32)) >> r.shm[tn];
        } else {
            v = requant_fast(acc[tm][tn][i] + r.bias[tn], r.mul[tn], r.rnd[tn], r.shm[tn]);
        }
        if (RES) v += (int)(signed char)(rr >> (8 * tn));
        q[tn] = RELU ? min(max(v, 0), 127) : min(max(v, -128), 127);
    }
    return pack4(q[0], q[1], q[2], q[3]);
}

// The fields of the chosen mode only, 16 registers for a lane's four channels (a kernel that keeps
// several channel sets resident across a loop cannot afford RqLane's 28):
//   mode 0: a = bias, b = shift
//   mode 1: (b, a) = the 64-bit addend bias*mult + 2^(30+shift) (high, low word), s = shift - 1
//   mode 2: a = bias, b = 2^(shift-2), s = shift - 1
// and m = mult in every mode.
struct RqPacked {
    int m[4], a[4], b[4], s[4];
};

__device__ __forceinline__ RqPacked rq_pack(const RqLane &r, int mode)
{
    RqPacked p;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        p.m[j] = r.mul[j];
        p.a[j] = mode == 1 ? (int)(unsigned)r.add[j] : r.bias[j];
        p.b[j] = mode == 0 ? r.shf[j] : (mode == 1 ? (int)(r.add[j] >> 32) : r.rnd[j]);
        p.s[j] = r.shm[j];
    }
    return p;
}

// Channel j of a packed set applied to one accumulator (mode MODE, no clamp).
template <int MODE>
__device__ __forceinline__ int rq_apply(int acc, const RqPacked &p, int j)
{
    if (MODE == 0) return requant_any(acc + p.a[j], p.m[j], p.b[j]);
    if (MODE == 1) {
        const long long add = (long long)(((unsigned long long)(unsigned)p.b[j] << 32) | (unsigned)p.a[j]);
        const long long q = (long long)acc * (long long)p.m[j] + add;
        return ((int)(q >> 32)) >> p.s[j];
    }
    return requant_fast(acc + p.a[j], p.m[j], p.b[j], p.s[j]);
}

// requant_row with a packed set: the lane's 4 channels of row 16tm + 4i + g.
template <int MODE, bool RES, bool RELU>
__device__ __forceinline__ unsigned requant_row_p(const v4i (&acc)[4][4], int tm, int i, const RqPacked &p,
                                                  unsigned rr)
{
    int q[4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
        int v = rq_apply<MODE>(acc[tm][tn][i], p, tn);
        if (RES) v += (int)(signed char)(rr >> (8 * tn));
        q[tn] = RELU ? min(max(v, 0), 127) : min(max(v, -128), 127);
    }
    return pack4(q[0], q[1], q[2], q[3]);
}

// Four channels of one output pixel (channel j of the set in acc[j]) requantised, no shortcut,
// clamped (ReLU or not) and packed into one word.
template <int MODE, bool RELU>
__device__ __forceinline__ unsigned requant_quad_p(v4i acc, const RqPacked &p)
{
    int q[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int v = rq_apply<MODE>(acc[j], p, j);
        q[j] = RELU ? min(max(v, 0), 127) : min(max(v, -128), 127);
    }
    return pack4(q[0], q[1], q[2], q[3]);
}

// Requantise a wave's (16 TM)x64 accumulator tile into the LDS staging tile (row stride BN),
// adding the shortcut bytes already there when RES.  Lane (g, c) owns tile rows
// 16tm + 4i + g and the 4 bytes at column 4c.
template <int MODE, bool RES, bool RELU, int BN, int TM>
__device__ __forceinline__ void requant_tile(const v4i (&acc)[TM][4], int8_t *rbase, const RqLane &r)
{
#pragma unroll
    for (int tm = 0; tm < TM; ++tm)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            unsigned *rp = (unsigned *)(rbase + (16 * tm + 4 * i) * BN);
            *rp = requant_row<MODE, RES, RELU>(acc, tm, i, r, RES ? *rp : 0u);
        }
}

// The three modes dispatched on rq_setup's wave-uniform choice.
template <bool RES, bool RELU, int BN, int TM>
__device__ __forceinline__ void requant_tile_any(int mode, const v4i (&acc)[TM][4], int8_t *rbase, const RqLane &r)
{
    if (mode == 0)
        requant_tile<0, RES, RELU, BN>(acc, rbase, r);
    else if (mode == 1)
        requant_tile<1, RES, RELU, BN>(acc, rbase, r);
    else
        requant_tile<2, RES, RELU, BN>(acc, rbase, r);
}

// A lane's 16 requantised rows kept in registers (a shortcut that never leaves the lane):
// sc[tm][i] holds the 4 bytes of row 16tm + 4i + g, no ReLU, no shortcut of its own.
template <int MODE>
__device__ __forceinline__ void requant_regs(const v4i (&acc)[4][4], const RqLane &r, unsigned (&sc)[4][4])
{
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int i = 0; i < 4; ++i) sc[tm][i] = requant_row<MODE, false, false>(acc, tm, i, r, 0u);
}

__device__ __forceinline__ void requant_regs_any(int mode, const v4i (&acc)[4][4], const RqLane &r,
                                                 unsigned (&sc)[4][4])
{
    if (mode == 0)
        requant_regs<0>(acc, r, sc);
    else if (mode == 1)
        requant_regs<1>(acc, r, sc);
    else
        requant_regs<2>(acc, r, sc);
}

// The final requantisation with the shortcut taken from registers (sc as requant_regs leaves
// it), written to the LDS staging tile (row stride BN).
template <int MODE, bool RELU, int BN>
__device__ __forceinline__ void requant_tile_sc(const v4i (&acc)[4][4], int8_t *rbase, const RqLane &r,
                                                const unsigned (&sc)[4][4])
{
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int i = 0; i < 4; ++i)
            *(unsigned *)(rbase + (16 * tm + 4 * i) * BN) = requant_row<MODE, true, RELU>(acc, tm, i, r, sc[tm][i]);
}

template <bool RELU, int BN>
__device__ __forceinline__ void requant_tile_sc_any(int mode, const v4i (&acc)[4][4], int8_t *rbase,
                                                    const RqLane &r, const unsigned (&sc)[4][4])
{
    if (mode == 0)
        requant_tile_sc<0, RELU, BN>(acc, rbase, r, sc);
    else if (mode == 1)
        requant_tile_sc<1, RELU, BN>(acc, rbase, r, sc);
    else
        requant_tile_sc<2, RELU, BN>(acc, rbase, r, sc);
}

}  // namespace ifx
