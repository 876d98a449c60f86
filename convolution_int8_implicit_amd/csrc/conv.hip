// Implicit-GEMM int8 convolution with the fused requant / shortcut / ReLU
// epilogue, for gfx950 (CDNA4) int8 MFMA.
//
// What is computed (Inspur conv-merge article, section 3.3): the convolution
// is the matrix product data[M,K] . weight[N,K]^T with M = batch*Ho*Wo output
// pixels, N = output channels and K = KH*KW*Ic, both operands K-contiguous
// thanks to the NC/32HW32 activation and [O1,KH,KW,I1,O2,32] weight layouts
// (section 3.1).  The epilogue (section 3.4: BN, Sum with the shortcut, ReLU)
// runs on the int32 accumulators before anything is written, and the
// shortcut tile is fetched at kernel start so its latency hides behind the
// contraction (the article's early asynchronous shortcut copy).
//
// gfx950 design (not the article's A100 tiling):
//   * one 256-thread workgroup (4 wave64s) owns a BM x BN output tile; each
//     wave owns 64x64 = 4x4 tiles of v_mfma_i32_16x16x64_i8;
//   * the K loop steps 64 bytes (two 32-channel blocks) at a time through an
//     ST-deep LDS ring filled by direct buffer->LDS 16-byte loads
//     (buffer_load_dwordx4 ... lds): loads for step k+ST-1 are in flight
//     while the MFMAs consume step k, with no register staging; the buffer
//     range check turns every out-of-image tap, ragged row or padded channel
//     into zeros, so the implicit GEMM needs no im2col and no branches;
//   * LDS rows are 64 bytes with an XOR swizzle of the four 16-byte chunks,
//     realised by choosing which global chunk each lane fetches;
//   * MFMA columns are permuted so that each lane holds four consecutive
//     output channels of a pixel: the epilogue requantises in registers,
//     stages the packed bytes through LDS and writes whole 16-byte chunks of
//     the NC/32HW32 output (the shortcut arrives the same way);
//   * the BN bias is folded into the accumulator initial value;
//   * workgroups are renumbered so that tiles sharing an activation tile run
//     back to back on the same XCD (own L2).
#include "ifx_internal.h"

typedef int ifx_v4i __attribute__((ext_vector_type(4)));

// Direct buffer -> LDS load: each lane's `size` bytes land at lds + lane * size.
__device__ void ifx_raw_buffer_load_lds(ifx_v4i rsrc, __attribute__((address_space(3))) void *lds, int size,
                                        unsigned voffset, int soffset, int offset,
                                        int aux) __asm("llvm.amdgcn.raw.buffer.load.lds");

namespace ifx {
namespace {

typedef ifx_v4i v4i;

constexpr int kThreads = 256;
constexpr int kStages = 4;
constexpr unsigned kOOB = 0x80000000u;  // offset past every buffer range: loads return zero


// Buffer resource (gfx9 layout): 48-bit base, stride 0, byte range, raw-buffer config word.
__device__ __forceinline__ v4i make_rsrc(const void *base, unsigned range)
{
    unsigned long long a = (unsigned long long)base;
    v4i r;
    r.x = __builtin_amdgcn_readfirstlane((int)(unsigned)a);
    r.y = __builtin_amdgcn_readfirstlane((int)(unsigned)(a >> 32) & 0xffff);
    r.z = __builtin_amdgcn_readfirstlane((int)range);
    r.w = 0x00020000;
    return r;
}

__device__ __forceinline__ void load16_lds(v4i rsrc, int8_t *lds_wave_base, unsigned voff)
{
    ifx_raw_buffer_load_lds(rsrc, (__attribute__((address_space(3))) void *)(lds_wave_base), 16, voff, 0, 0, 0);
}

// s_waitcnt vmcnt(n) with expcnt/lgkmcnt left unconstrained (gfx9 encoding).
template <int N>
__device__ __forceinline__ void wait_vmcnt()
{
    static_assert(N >= 0 && N < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((N & 0xf) | ((N >> 4) << 14) | (0x7 << 4) | (0xf << 8));
}

// Workgroup barrier for the LDS ring.  Each wave first waits for its own
// direct-to-LDS loads of the stage (wait_vmcnt); LDS needs no cache
// maintenance, so a bare s_barrier then makes every wave's stage data visible.
// (__syncthreads would add a release fence that drains all loads in flight,
// i.e. the whole ring.)  The empty asm keeps the compiler from moving LDS
// accesses across the barrier.
__device__ __forceinline__ void ring_barrier()
{
    asm volatile("" ::: "memory");
    __builtin_amdgcn_s_barrier();
    asm volatile("" ::: "memory");
}

// 16-byte-chunk XOR swizzle of a 64-byte LDS row: conflict-free ds_read_b128
// for both the row-major operand fetch and the permuted pixel order.
__device__ __forceinline__ int swz(int row) { return ((row >> 1) ^ (row >> 3)) & 3; }

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

// sh >= 2 and a ReLU with no shortcut: for y < 0 the result is <= 0 either way
// and the ReLU clears it, so the [y<0] tie correction can be dropped.
__device__ __forceinline__ int requant_relu(int y, int m, int rnd_hi, int sh_m1)
{
    long long add = (long long)((unsigned long long)(unsigned)rnd_hi << 32);
    long long p = (long long)y * (long long)m + add;
    return ((int)(p >> 32)) >> sh_m1;
}

// Requantise a wave's 64x64 accumulator tile and leave the packed int8 bytes
// in the LDS staging tile (row stride BN), adding the shortcut bytes already
// there when RES.  MODE 0: general (any shift); 1: shift >= 2 with ReLU and no
// shortcut; 2: shift >= 2.  Lane (g, c) owns pixel rows 16tm + 4i + g and the
// 4 bytes at column 4c.
template <int MODE, bool RES, int BN>
__device__ __forceinline__ void requant_tile(const v4i (&acc)[4][4], int8_t *rbase, const int (&mul)[4],
                                             const int (&rnd)[4], const int (&shm)[4], const int (&shf)[4],
                                             const int (&keep)[4], bool relu)
{
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            unsigned *rp = (unsigned *)(rbase + (16 * tm + 4 * i) * BN);
            const unsigned rr = RES ? *rp : 0u;
            unsigned packed = 0;
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) {
                const int yv = acc[tm][tn][i];
                int q;
                if (MODE == 0)
                    q = requant_any(yv, mul[tn], shf[tn]);
                else if (MODE == 1)
                    q = requant_relu(yv, mul[tn], rnd[tn], shm[tn]);
                else
                    q = requant_fast(yv, mul[tn], rnd[tn], shm[tn]);
                if (RES) q += (int)(signed char)(rr >> (8 * tn));
                q = relu ? min(max(q, 0), 127) : min(max(q, -128), 127);
                packed |= (unsigned)(q & keep[tn]) << (8 * tn);
            }
            *rp = packed;
        }
}

template <int KH, int KW, int BM, int BN, bool RES>
struct ConvCfg {
    static constexpr int WAVES_M = BM / 64;
    static constexpr int WAVES_N = BN / 64;
    static_assert(WAVES_M * WAVES_N == kThreads / 64, "4 waves per workgroup");
    static constexpr int AI = BM * 64 / 16 / kThreads;  // A-tile loads per thread per stage
    static constexpr int BI = BN * 64 / 16 / kThreads;  // B-tile loads per thread per stage
    static constexpr int STAGE = (BM + BN) * 64;        // bytes per ring stage
    static constexpr int RI = BM * BN / 16 / kThreads;  // shortcut loads per thread
    static constexpr int RING = kStages * STAGE;
    static constexpr int LDS = RES ? RING + BM * BN : (RING > BM * BN ? RING : BM * BN);
};

template <int KH, int KW, int BM, int BN, bool RES>
__global__ __launch_bounds__(kThreads, 2) void conv_kernel(ConvArgs a)
{
    using C = ConvCfg<KH, KW, BM, BN, RES>;
    constexpr int AI = C::AI, BI = C::BI, STAGE = C::STAGE;
    __shared__ __attribute__((aligned(1024))) int8_t smem[C::LDS];
    int8_t *R = RES ? smem + C::RING : smem;  // [BM][BN] shortcut / output staging

    const int tid = threadIdx.x;
    const int lane = tid & 63;
    const int wave = tid >> 6;
    const int wm0 = (wave % C::WAVES_M) * 64;
    const int wn0 = (wave / C::WAVES_M) * 64;

    // ---- tile of this workgroup (XCD-aware renumbering) ----
    const int tiles_n = (a.oc1 * 32 + BN - 1) / BN;
    const int G = gridDim.x;
    const int bid = blockIdx.x;
    const int per_xcd = G >> 3;
    const int lin = bid < (per_xcd << 3) ? (bid & 7) * per_xcd + (bid >> 3) : bid;
    const int tile_n = lin % tiles_n;
    const int tile_m = lin / tiles_n;
    const int m0 = tile_m * BM;
    const int n0 = tile_n * BN;

    const int HoWo = a.ho * a.wo;
    const int HW = a.h * a.w;
    const int img0 = m0 / HoWo;  // first image touched by this tile

    // per-lane output channels and their folded BN bias (loaded before any
    // ring traffic so waiting for them never drains the prefetches)
    const int c = lane & 15;
    const int g = lane >> 4;
    const int ocl = n0 + wn0 + 4 * c;  // first of this lane's four output channels
    int bias_v[4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) bias_v[tn] = (ocl + tn < a.oc) ? a.bias[ocl + tn] : 0;

    // ---- buffer resources, based at the tile's first image (offsets < 2^31) ----
    const long long in_img = (long long)a.i1 * HW * 32;
    const long long in_total = (long long)a.n * in_img;
    const long long in_base = (long long)img0 * in_img;
    const unsigned in_range = (unsigned)min(in_total - in_base, 0x7ffffff0ll);
    const v4i rsA = make_rsrc(a.x + in_base, in_range);
    const long long wbytes = (long long)((a.oc + a.o2 - 1) / a.o2) * a.o2 * KH * KW * a.i1 * 32;
    const v4i rsB = make_rsrc(a.wt, (unsigned)min(wbytes, 0x7ffffff0ll));

    // ---- shortcut tile -> LDS (issued first; lands while the K loop runs) ----
    if (RES) {
        const long long out_img = (long long)a.oc1 * HoWo * 32;
        const long long r_base = (long long)img0 * out_img;
        const unsigned r_range = (unsigned)min((long long)a.n * out_img - r_base, 0x7ffffff0ll);
        const v4i rsR = make_rsrc(a.res + r_base, r_range);
        constexpr int CPR = BN / 16;  // 16-byte chunks per staged row
#pragma unroll
        for (int j = 0; j < C::RI; ++j) {
            const int slot = (j * 4 + wave) * 64 + lane;  // 16-byte slot of R
            const int row = slot / CPR, ch = slot % CPR;
            const int p = m0 + row;
            const int oc = n0 + ch * 16;
            unsigned off = kOOB;
            if (p < a.m && oc < a.oc1 * 32) {
                const int b = p / HoWo, hw = p - (p / HoWo) * HoWo;
                off = (unsigned)((((long long)(b - img0) * a.oc1 + (oc >> 5)) * HoWo + hw) * 32 + (oc & 31));
            }
            load16_lds(rsR, R + (j * 4 + wave) * 1024, off);
        }
    }

    // ---- per-lane load plans for the A (activation) and B (weight) tiles ----
    // A: instruction j of wave w fills rows [(4j+w)*16, +16) of the stage;
    //    lane l -> row (4j+w)*16 + l/4, physical chunk l%4.
    unsigned a_img[AI];
    int a_iy[AI], a_ix[AI], a_sel[AI];
    bool a_ok[AI];
#pragma unroll
    for (int j = 0; j < AI; ++j) {
        const int row = (j * 4 + wave) * 16 + (lane >> 2);
        const int lch = (lane & 3) ^ swz(row);
        const int p = m0 + row;
        a_ok[j] = p < a.m;
        const int pp = a_ok[j] ? p : m0;
        const int b = pp / HoWo;
        const int rem = pp - b * HoWo;
        const int oy = rem / a.wo;
        const int ox = rem - oy * a.wo;
        a_iy[j] = oy * a.stride - a.pad;
        a_ix[j] = ox * a.stride - a.pad;
        a_img[j] = (unsigned)((long long)(b - img0) * in_img) + (lch & 1) * 16;
        a_sel[j] = lch >> 1;  // which of the step's two 32-channel blocks
    }
    // B: instruction j of wave w fills physical rows [(4j+w)*16, +16); within
    //    each 64-row group physical row r holds output channel (r%16)*4 + r/16.
    unsigned b_off[BI];
    int b_sel[BI];
    bool b_ok[BI];
#pragma unroll
    for (int j = 0; j < BI; ++j) {
        const int prow = (j * 4 + wave) * 16 + (lane >> 2);
        const int lch = (lane & 3) ^ swz(prow);
        const int o = (prow & ~63) + (prow & 15) * 4 + ((prow & 63) >> 4);
        const int R_ = n0 + o;
        const int wrows = ((a.oc + a.o2 - 1) / a.o2) * a.o2;
        b_ok[j] = R_ < wrows;
        const int RR = b_ok[j] ? R_ : 0;
        const int o1 = RR / a.o2, o2i = RR - (RR / a.o2) * a.o2;
        b_off[j] = (unsigned)(((long long)o1 * KH * KW * a.i1 * a.o2 + o2i) * 32) + (lch & 1) * 16;
        b_sel[j] = lch >> 1;
    }

    const int nsteps = (a.nkb + 1) >> 1;
    const unsigned wstride_c1 = (unsigned)a.o2 * 32;

    // uniform reduction position of the step's first block: (ky, kx, c1)
    int s_c1 = 0, s_kx = 0, s_ky = 0, s_kb = 0;
    auto issue = [&](int slot) {
        // second block of the step: the block after (ky, kx, c1)
        int c1b = s_c1 + 1, kxb = s_kx, kyb = s_ky;
        if (c1b == a.i1) {
            c1b = 0;
            if (++kxb == KW) {
                kxb = 0;
                ++kyb;
            }
        }
        int8_t *st = smem + slot * STAGE;
#pragma unroll
        for (int j = 0; j < AI; ++j) {
            const int sel = a_sel[j];
            const int c1 = sel ? c1b : s_c1;
            const int kx = sel ? kxb : s_kx;
            const int ky = sel ? kyb : s_ky;
            const int iy = a_iy[j] + ky, ix = a_ix[j] + kx;
            bool ok = a_ok[j] && (s_kb + sel) < a.nkb;
            if (KH > 1) ok = ok && (unsigned)iy < (unsigned)a.h;
            if (KW > 1) ok = ok && (unsigned)ix < (unsigned)a.w;
            const unsigned off = ok ? a_img[j] + (unsigned)(((c1 * a.h + iy) * a.w + ix) * 32) : kOOB;
            load16_lds(rsA, st + (j * 4 + wave) * 1024, off);
        }
#pragma unroll
        for (int j = 0; j < BI; ++j) {
            const int sel = b_sel[j];
            const int c1 = sel ? c1b : s_c1;
            const int kx = sel ? kxb : s_kx;
            const int ky = sel ? kyb : s_ky;
            const bool ok = b_ok[j] && (s_kb + sel) < a.nkb;
            const unsigned off = ok ? b_off[j] + (unsigned)((ky * KW + kx) * a.i1 + c1) * wstride_c1 : kOOB;
            load16_lds(rsB, st + BM * 64 + (j * 4 + wave) * 1024, off);
        }
        // advance two blocks
        s_kb += 2;
        s_c1 += 2;
        while (s_c1 >= a.i1) {
            s_c1 -= a.i1;
            if (++s_kx == KW) {
                s_kx = 0;
                ++s_ky;
            }
        }
    };

    // ---- accumulators, initialised with the folded BN bias ----
    v4i acc[4][4];
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) acc[tm][tn] = (v4i){bias_v[tn], bias_v[tn], bias_v[tn], bias_v[tn]};
    }

    // ---- K loop over the LDS ring ----
#pragma unroll
    for (int s = 0; s < kStages - 1; ++s) issue(s);
    for (int step = 0; step < nsteps; ++step) {
        wait_vmcnt<(kStages - 2) * (AI + BI)>();
        ring_barrier();
        issue((step + kStages - 1) % kStages);  // past the end: all lanes out of range (zeros)
        const int8_t *st = smem + (step % kStages) * STAGE;
        v4i af[4], bf[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            const int r = lane & 15;
            const int row = wm0 + 16 * tm + 4 * (r & 3) + (r >> 2);
            af[tm] = *(const v4i *)(st + row * 64 + ((g ^ swz(row)) << 4));
        }
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            const int row = wn0 + 16 * tn + c;
            bf[tn] = *(const v4i *)(st + BM * 64 + row * 64 + ((g ^ swz(row)) << 4));
        }
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
                acc[tm][tn] = __builtin_amdgcn_mfma_i32_16x16x64_i8(af[tm], bf[tn], acc[tm][tn], 0, 0, 0);
    }
    wait_vmcnt<0>();
    __syncthreads();

    // ---- fused epilogue ----
    // lane (g, c) of MFMA tile (tm, tn) holds pixel wm0 + 16tm + 4i + g of the
    // tile and output channel ocl + tn, for i = 0..3.
    const int pbase = m0 + wm0;
    if (a.out_i32) {
        int32_t *y = (int32_t *)a.y;
        const bool vec = (a.oc & 3) == 0 && ocl + 3 < a.oc;
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int i = 0; i < 4; ++i) {
                const int p = pbase + 16 * tm + 4 * i + g;
                if (p >= a.m) continue;
                const long long off = (long long)p * a.oc + ocl;
                if (vec) {
                    *(v4i *)(y + off) = (v4i){acc[tm][0][i], acc[tm][1][i], acc[tm][2][i], acc[tm][3][i]};
                } else {
#pragma unroll
                    for (int tn = 0; tn < 4; ++tn)
                        if (ocl + tn < a.oc) y[off + tn] = acc[tm][tn][i];
                }
            }
        return;
    }

    int mul[4], rnd[4], shm[4], shf[4], keep[4];
    bool fast_lane = true;
#pragma unroll
    for (int tn = 0; tn < 4; ++tn) {
        const int o = ocl + tn;
        const bool v = o < a.oc;
        mul[tn] = v ? a.mult[o] : 0;
        shf[tn] = v ? a.shift[o] : 2;
        fast_lane = fast_lane && shf[tn] >= 2;
        rnd[tn] = 1 << ((shf[tn] - 2) & 31);
        shm[tn] = shf[tn] - 1;
        keep[tn] = v ? 0xff : 0;
    }
    const bool fast = __all(fast_lane);
    const bool relu = a.relu != 0;

    // requantise in registers; shortcut bytes and results share the staging tile R
    int8_t *rbase = R + (wm0 + g) * BN + wn0 + 4 * c;
    if (!fast)
        requant_tile<0, RES, BN>(acc, rbase, mul, rnd, shm, shf, keep, relu);
    else if (!RES && relu)
        requant_tile<1, RES, BN>(acc, rbase, mul, rnd, shm, shf, keep, relu);
    else
        requant_tile<2, RES, BN>(acc, rbase, mul, rnd, shm, shf, keep, relu);
    __syncthreads();

    // 16-byte stores of the wave's 64 pixels x 64 channels
    int8_t *y = (int8_t *)a.y;
    const int k = lane & 3;
    const int och = n0 + wn0 + 16 * k;  // first channel of this lane's chunk
    if (och >= a.oc1 * 32) return;
    const int b0 = pbase / HoWo;
    const int hw0 = pbase - b0 * HoWo;
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int prow = 16 * j + (lane >> 2);
        if (pbase + prow >= a.m) break;
        int b = b0, hw = hw0 + prow;
        while (hw >= HoWo) {
            hw -= HoWo;
            ++b;
        }
        const v4i v = *(const v4i *)(R + (wm0 + prow) * BN + wn0 + 16 * k);
        *(v4i *)(y + (((long long)b * a.oc1 + (och >> 5)) * HoWo + hw) * 32 + (och & 31)) = v;
    }
}

template <int KH, int KW, int BM, int BN>
hipError_t launch_tiles(const ConvArgs &a, hipStream_t s)
{
    const long long tiles_m = (a.m + BM - 1) / BM;
    const long long tiles_n = (a.oc1 * 32 + BN - 1) / BN;
    const long long blocks = tiles_m * tiles_n;
    if (blocks <= 0) return hipSuccess;
    if (blocks > 0x7fffffffLL) return hipErrorInvalidConfiguration;
    if (a.residual)
        hipLaunchKernelGGL((conv_kernel<KH, KW, BM, BN, true>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    else
        hipLaunchKernelGGL((conv_kernel<KH, KW, BM, BN, false>), dim3((unsigned)blocks), dim3(kThreads), 0, s, a);
    return hipGetLastError();
}

template <int KH, int KW>
hipError_t launch_k(const ConvArgs &a, hipStream_t s)
{
    if (a.oc1 * 32 > 64) return launch_tiles<KH, KW, 128, 128>(a, s);
    return launch_tiles<KH, KW, 256, 64>(a, s);
}

}  // namespace

hipError_t launch_conv(const ConvArgs &a, int kh, int kw, hipStream_t s)
{
    if (kh == 1 && kw == 1) return launch_k<1, 1>(a, s);
    if (kh == 3 && kw == 3) return launch_k<3, 3>(a, s);
    return hipErrorInvalidValue;
}

}  // namespace ifx
